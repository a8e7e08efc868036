// One-token weight streams of the dense products (bf16, m = 1): y = A v for
// a row-major A, every weight byte read once, in contiguous per-workgroup
// blocks of whole rows, with every load of a wave in flight before the first
// is used.
//
// A workgroup of 8 waves owns rpb consecutive rows; each row is cut into
// items of `seg` elements (a multiple of 512: one 16-byte chunk per lane per
// 512), one item per wave, so a wave's loads (up to 8 chunks per lane, plus a
// short gate row riding along) all go out before it computes, and few
// registers leave room for three workgroups per CU. The vectors (x or h bf16,
// the low-rank t fp32) are staged once per workgroup in LDS while the weight
// loads fly. Per item a lane dots its chunks in order (bf16 pairs with
// v_dot2_f32_bf16), a wave butterfly sums the lanes, and the epilogue adds a
// row's items in order:
//   EPI_OUT   fp32 row values (t = V x)
//   EPI_Y     y rows (bf16 or fp32)
//   EPI_HID   h = a(z) u of the dense FFN: a second matrix per row gives the
//             gate (W_gate with x, or the low-rank U with t), z = g + b, and
//             the activation keeps the selection's elementwise mask (LoPA
//             page, "How LoPA Gating Restructures FFN Computation": gate
//             projection, activation, elementwise product)
//   EPI_SCORE the WINA score of every neuron, s = |a(z) u| c (WINA page,
//             section 3.1), with h, into the top-k kernel's buffers
#include "common.cuh"
#include "kernels.cuh"
#include "wave.cuh"

namespace ffn {

namespace {

constexpr int kSgWaves = 8;
constexpr int kSgThreads = 64 * kSgWaves;
constexpr int kSgMaxVec = 8 * 8 * kSgThreads;      // bf16 vector elements staged (8 chunks a thread)
constexpr int kSgRideMax = 1024;                   // a gate row this short rides with the row's first item

__device__ __forceinline__ float sg_act(int act, float z) { return act == ACT_RELU ? fmaxf(z, 0.f) : z / (1.f + expf(-z)); }

}  // namespace

// Item i of the workgroup (one per wave): row i / ipr, segment i % ipr. With
// a short gate (NPG > 0: Kg <= 512 NPG) the gate row's chunks ride with
// segment 0 of the main row; a gate as long as the main row (the full W_gate
// with x) has segments of its own after the main ones.
template <int VB, int NPG>
__global__ __launch_bounds__(kSgThreads) void k_sgemv1(const Sgemv1Desc d) {
  extern __shared__ uint4 s_dyn[];                 // bf16 vector [kvec], then fp32 gate vector [Kg]
  __shared__ float s_part[kSgWaves];
  __shared__ float s_gpart[kSgWaves];
  const int lane = lane_id(), wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int sm = (d.K + d.seg - 1) / d.seg;                      // main segments per row
  const int sg = (d.Ag && NPG == 0) ? (d.Kg + d.seg - 1) / d.seg : 0;
  const int ipr = sm + sg;
  const int row0 = blockIdx.x * d.rpb;
  const int nrow = min(d.rpb, d.N - row0);
  const int np = d.seg / 512;
  uint16_t* s_vec = reinterpret_cast<uint16_t*>(s_dyn);
  float* s_vg = reinterpret_cast<float*>(reinterpret_cast<char*>(s_dyn) + (size_t)d.kvec * 2);

  // the vectors' loads first (their LDS stores then wait for them only)
  uint4 vv[VB];
#pragma unroll
  for (int i = 0; i < VB; ++i) {
    const int c = tid + i * kSgThreads;
    vv[i] = c < d.kvec / 8 ? ldg16(d.vec + (size_t)c * 8) : uint4{0, 0, 0, 0};
  }
  constexpr int GV = NPG > 0 ? (512 * NPG / 4 + kSgThreads - 1) / kSgThreads : 1;   // fp32 gate-vector float4s a thread
  float4 vg[GV];
#pragma unroll
  for (int i = 0; i < GV; ++i) {
    const int c = tid + i * kSgThreads;
    vg[i] = (NPG > 0 && d.vecg && c < d.Kg / 4) ? *reinterpret_cast<const float4*>(d.vecg + (size_t)c * 4)
                                                : float4{0.f, 0.f, 0.f, 0.f};
  }

  // this wave's item
  const int i = wave;
  const bool live = i < nrow * ipr;
  const int r = live ? i / ipr : 0, s = i - r * ipr;
  const bool gseg = s >= sm;                                       // a segment of a long gate row
  const int seg = gseg ? s - sm : s;
  const uint16_t* A = gseg ? d.Ag : d.A;
  const int klen = gseg ? d.Kg : d.K;
  const int col0 = seg * d.seg;
  const uint16_t* rp = A + (size_t)(row0 + r) * klen;
  uint4 a[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int col = col0 + p * 512 + lane * 8;
    a[p] = (live && p < np && col < klen) ? ldg16(rp + col) : uint4{0, 0, 0, 0};
  }
  uint4 ag[NPG > 0 ? NPG : 1];
  const bool ride = NPG > 0 && live && !gseg && seg == 0;
  if constexpr (NPG > 0) {
    const uint16_t* gp = d.Ag + (size_t)(row0 + r) * d.Kg;
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      const int col = p * 512 + lane * 8;
      ag[p] = (ride && col < d.Kg) ? ldg16(gp + col) : uint4{0, 0, 0, 0};
    }
  }

#pragma unroll
  for (int k = 0; k < VB; ++k) {
    const int c = tid + k * kSgThreads;
    if (c < d.kvec / 8) reinterpret_cast<uint4*>(s_vec)[c] = vv[k];
  }
  if constexpr (NPG > 0) {
#pragma unroll
    for (int k = 0; k < GV; ++k) {
      const int c = tid + k * kSgThreads;
      if (c < d.Kg / 4) reinterpret_cast<float4*>(s_vg)[c] = vg[k];
    }
  }
  __syncthreads();

  if (live) {
    // main (or long gate) segment against the bf16 vector
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int col = col0 + p * 512 + lane * 8;
      if (p < np && col < klen) acc = dot8_bf_d2(a[p], *reinterpret_cast<const uint4*>(s_vec + col), acc);
    }
    acc = wave_sum(acc);
    float gacc = 0.f;
    if constexpr (NPG > 0) {
      if (ride) {                                // the short gate row against t (fp32)
#pragma unroll
        for (int p = 0; p < NPG; ++p) {
          const int col = p * 512 + lane * 8;
          if (col < d.Kg) {
            const float4 t0 = *reinterpret_cast<const float4*>(s_vg + col);
            const float4 t1 = *reinterpret_cast<const float4*>(s_vg + col + 4);
            gacc = dot8_f32(ag[p], t0, t1, gacc);
          }
        }
        gacc = wave_sum(gacc);
      }
    }
    if (lane == 0) {
      s_part[wave] = acc;
      s_gpart[wave] = gacc;
    }
  }
  __syncthreads();

  if (tid < nrow) {
    const int rr = tid, row = row0 + rr;
    float u = 0.f, g = 0.f;
    for (int q = 0; q < sm; ++q) u += s_part[rr * ipr + q];
    if (NPG > 0) g = s_gpart[rr * ipr];
    for (int q = 0; q < sg; ++q) g += s_part[rr * ipr + sm + q];
    if (d.epi == SG_OUT) {
      d.out[row] = u;
    } else if (d.epi == SG_Y) {
      if (d.y_f32) reinterpret_cast<float*>(d.y)[row] = u;
      else reinterpret_cast<uint16_t*>(d.y)[row] = (uint16_t)f2bf(u);
    } else {
      const float b = d.bias ? d.bias[0] : d.bias_scalar;
      const float z = g + b;
      if (d.epi == SG_HID) {
        float av;
        if (d.sel == SEL_TOPK) av = sg_act(d.act, z);
        else av = z > (d.sel == SEL_THRESH ? fmaxf(d.tau[0], 0.f) : 0.f) ? z : 0.f;
        reinterpret_cast<uint16_t*>(d.hout)[row] = (uint16_t)f2bf(av * u);
      } else {                                       // SG_SCORE
        const float h = sg_act(d.act, z) * u;
        const float sc = fabsf(h) * d.colnorm[row];
        d.s_buf[row] = sc;
        d.h_buf[row] = h;
        if (d.g_debug) d.g_debug[row] = g;
        if (d.s_debug) d.s_debug[row] = sc;
      }
    }
  }
}

// Short gate rows (the low-rank U, Kg <= 1024 with an fp32 vector) ride with
// the main row's first item; otherwise the gate has its own segments.
static int sg_npg(const Sgemv1Desc& d) {
  if (!d.Ag || !d.vecg || d.Kg > kSgRideMax) return 0;
  return d.Kg <= 512 ? 1 : 2;
}

bool sgemv1_plan(Sgemv1Desc& d, int cus) {
  if (d.N < 1 || d.K < 8 || d.K % 8 != 0 || !d.A || !d.vec) return false;
  if (d.Ag && (d.Kg < 8 || d.Kg % 8 != 0)) return false;
  if (d.vecg && sg_npg(d) == 0) return false;      // an fp32 gate vector only as a short ride-along row
  const bool long_gate = d.Ag && sg_npg(d) == 0;
  if (long_gate && d.Kg != d.K) return false;      // a full gate shares the bf16 vector
  // item size: 4096 elements, or smaller until there is an item for every
  // wave of the chip (a short matrix such as V is otherwise read by too few)
  auto items = [&](int seg) { return (d.K + seg - 1) / seg + (long_gate ? (d.Kg + seg - 1) / seg : 0); };
  int seg = 4096;
  while (seg > 512 && (long long)d.N * items(seg) < 2LL * cus * kSgWaves) seg /= 2;
  const int ipr = items(seg);
  if (ipr > kSgWaves) return false;
  d.seg = seg;
  d.rpb = kSgWaves / ipr;                          // one item per wave
  d.kvec = (d.K + 7) / 8 * 8;
  if (d.kvec > kSgMaxVec) return false;
  return true;
}

size_t sgemv1_lds(const Sgemv1Desc& d) { return (size_t)d.kvec * 2 + (sg_npg(d) ? (size_t)d.Kg * 4 : 0); }

hipError_t launch_sgemv1(const Sgemv1Desc& d, hipStream_t s) {
  if (d.seg < 512 || d.seg % 512 != 0 || d.seg > 4096 || d.rpb < 1) return hipErrorInvalidValue;
  const int npg = sg_npg(d);
  const int ipr = (d.K + d.seg - 1) / d.seg + ((d.Ag && npg == 0) ? (d.Kg + d.seg - 1) / d.seg : 0);
  if (ipr * d.rpb > kSgWaves || d.kvec > kSgMaxVec) return hipErrorInvalidValue;
  const size_t lds = sgemv1_lds(d);
  const dim3 grid((d.N + d.rpb - 1) / d.rpb), blk(kSgThreads);
  const int chunks = (d.kvec / 8 + kSgThreads - 1) / kSgThreads;   // staging chunks per thread
  auto go = [&](auto kern) -> hipError_t {
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    ffn_launch(kern, grid, blk, lds, s, d);
    return hipGetLastError();
  };
  if (npg == 1) return chunks <= 1 ? go(k_sgemv1<1, 1>) : (chunks <= 2 ? go(k_sgemv1<2, 1>) : go(k_sgemv1<8, 1>));
  if (npg == 2) return chunks <= 1 ? go(k_sgemv1<1, 2>) : (chunks <= 2 ? go(k_sgemv1<2, 2>) : go(k_sgemv1<8, 2>));
  if (chunks <= 1) return go(k_sgemv1<1, 0>);
  if (chunks <= 2) return go(k_sgemv1<2, 0>);
  if (chunks <= 4) return go(k_sgemv1<4, 0>);
  if (chunks <= 8) return go(k_sgemv1<8, 0>);
  return hipErrorInvalidValue;
}

}  // namespace ffn
