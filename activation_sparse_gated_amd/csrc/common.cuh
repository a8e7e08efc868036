// Device helpers shared by the gfx950 kernels of the sparse gated FFN.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define FFN_WAVE 64

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace ffn {

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// 8 bf16 packed in a uint4 -> 8 floats (element e of the 16-byte chunk -> f[e]).
__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Copies n elements into LDS, element p from src(p), the block's threads
// taking elements in turn. Each thread issues up to NB loads before its first
// LDS store, so a pass costs one memory round trip per NB * blockDim elements
// (a plain strided copy loop waits for every load before the next).
// Loads past the end re-read element n - 1 (no branch around a load).
template <int NB, typename T, typename Src>
__device__ __forceinline__ void stage_lds(T* dst, int n, Src src) {
  for (int base = threadIdx.x; base < n; base += NB * blockDim.x) {
    T v[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) v[b] = src(min(base + b * (int)blockDim.x, n - 1));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int p = base + b * blockDim.x;
      if (p < n) dst[p] = v[b];
    }
  }
}

// ---------------------------------------------------------------- wave ops
// Exchange with a partner lane at butterfly level O (a power of two), all in
// the VALU: levels 1..8 as DPP moves, quad_perm [1,0,3,2] and [2,3,0,1] for
// 1 and 2, the half-row mirror (partner lane ^ 7) for 4 and the row mirror
// (lane ^ 15) for 8; levels 16 and 32 with gfx950's v_permlane16_swap /
// v_permlane32_swap on two copies of the value (the swap moves the odd
// 16-lane rows, or the upper 32 lanes, of one copy into the even rows, or
// lower lanes, of the other, so each lane finds its partner's value in one of
// the two results). A mirror partner differs from the lane in bit O and in lower bits only,
// so at each level it still pairs the lanes with bit O clear with those with
// it set, among lanes whose higher bits agree: butterfly reductions keep their
// lane-to-value mapping and sum every lane exactly once.
template <int O>
__device__ __forceinline__ int wave_xchg_i(int v) {
  if constexpr (O == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  else if constexpr (O == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  else if constexpr (O == 4) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  else if constexpr (O == 8) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  else if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? (int)r[0] : (int)r[1];
  } else {
    static_assert(O == 32, "butterfly level");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? (int)r[0] : (int)r[1];
  }
}
template <int O>
__device__ __forceinline__ float wave_xchg(float v) {
  return __int_as_float(wave_xchg_i<O>(__float_as_int(v)));
}

// Exact xor partner (lane ^ O), for butterflies over some lane bits only:
// DPP quad_perm for 1 and 2, the permlane swaps for 16 and 32, ds_bpermute
// for 4 and 8 (the row mirrors pair lane ^ 7 and lane ^ 15 there).
template <int O>
__device__ __forceinline__ float wave_xor(float v) {
  if constexpr (O == 4 || O == 8) return __shfl_xor(v, O, FFN_WAVE);
  else return wave_xchg<O>(v);
}

// Value of a wave-uniform lane `src` (a scalar read, no LDS round trip).
__device__ __forceinline__ int wave_read(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

// Butterfly sum: every lane ends with the same value (fp add is commutative
// and each level adds two lane groups that already agree).
__device__ __forceinline__ float wave_sum(float v) {
  v += wave_xchg<32>(v);
  v += wave_xchg<16>(v);
  v += wave_xchg<8>(v);
  v += wave_xchg<4>(v);
  v += wave_xchg<2>(v);
  v += wave_xchg<1>(v);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += wave_xchg_i<32>(v);
  v += wave_xchg_i<16>(v);
  v += wave_xchg_i<8>(v);
  v += wave_xchg_i<4>(v);
  v += wave_xchg_i<2>(v);
  v += wave_xchg_i<1>(v);
  return v;
}
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & (FFN_WAVE - 1); }
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Inclusive scan of ints across the wave (Hillis-Steele with shuffles).
// Inclusive scan across the wave in DPP moves: a Hillis-Steele scan inside
// each 16-lane row (row_shr 1, 2, 4, 8; lanes whose source lies before the row
// add 0), then row_bcast15 adds row 0's total to row 1 and row 2's to row 3,
// and row_bcast31 adds the first 32 lanes' total to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Exclusive scan over a block of NT threads (NT multiple of 64, <= 1024);
// `scratch` holds NT/64 ints. Returns the exclusive prefix; *total = sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int* total) {
  const int w = threadIdx.x / FFN_WAVE, l = lane_id();
  int inc = wave_incl_scan(v);
  if (l == 63) scratch[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / FFN_WAVE; ++i) {
    int s = scratch[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// ---------------------------------------------------------------- atomics
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store64_relaxed(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load64_relaxed(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-wide "last one out" ticket: every thread fences its prior global
// writes, thread 0 takes a ticket; returns true in the block that arrives last
// (which then sees every other block's writes). The counter is reset to 0 by
// that block, so it is ready for the next launch.
__device__ __forceinline__ bool block_last_arrival(uint32_t* counter, uint32_t total, int* s_flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = atomic_add_agent(counter, 1u);
    bool last = (t == total - 1);
    if (last) atomic_store_agent(counter, 0u);
    *s_flag = last ? 1 : 0;
  }
  __syncthreads();
  bool last = *s_flag != 0;
  if (last) __threadfence();
  return last;
}

// ---------------------------------------------------------------- control words
// Layout of the per-handle control block in the workspace (uint32 words).
enum CtrlWord : int {
  CTRL_EPOCH = 0,       // incremented once per gate pass; tags look-back words
  CTRL_GATE_DONE = 1,   // completion ticket of the gate kernel
  CTRL_VSTAGE_DONE = 2, // reserved
  CTRL_TOPK_DONE = 3,   // completion ticket of the top-k kernel
  CTRL_ERR = 4,         // nonzero once a bounded wait gave up (read by the host)
  CTRL_SPIN_LIMIT = 5,  // polls a wait makes before it gives up
  CTRL_WAIT_SKEW = 6,   // added to the epoch a wait expects (0; nonzero only to test the give-up path)
  CTRL_TILE_TICKETS = 64  // per-tile split-K tickets start here
};
constexpr uint32_t kDefaultSpinLimit = 1u << 20;   // about a second of polling

// What a waiting workgroup expects: the epoch its wait accepts and how many
// polls it may make. Read once per kernel from the control block.
struct WaitCtl {
  uint32_t want, limit;
};
__device__ __forceinline__ WaitCtl wait_ctl(const uint32_t* ctrl, uint32_t epoch) {
  const uint32_t skew = __hip_atomic_load(&ctrl[CTRL_WAIT_SKEW], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t limit = __hip_atomic_load(&ctrl[CTRL_SPIN_LIMIT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return WaitCtl{epoch + skew, limit};
}

// Bounded wait on an epoch-tagged 64-bit word (tag in the high half, a count
// or value in the low half), starting from an already loaded value w: polls
// until the tag equals wc.want. After wc.limit polls it gives up, raises the
// control block's error word (the host reads it through
// ffn_sparse_device_status) and returns the low half as it stands, so every
// wave still runs to the end of its kernel.
__device__ __forceinline__ uint32_t tagged_wait(const uint64_t* p, uint64_t w, const WaitCtl& wc, uint32_t* ctrl) {
  uint32_t n = 0;
  while ((uint32_t)(w >> 32) != wc.want) {
    if (++n > wc.limit) {
      __hip_atomic_store(&ctrl[CTRL_ERR], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    w = load64_relaxed(p);
  }
  return (uint32_t)w;
}

}  // namespace ffn
