// Fused sparse up + down projection over the TwELL pack, and routing.
//
// For every packed neuron i of token t: u_i = <W_up[i, :], x_t>,
// h_i = a_i * u_i (top-k packs already hold h_i), y_t += h_i * W_down[:, i].
// Both weight rows are contiguous (W_up is neuron-major; W_down is kept
// neuron-major in the workspace), so a wave gathers each with 16-byte loads
// covering 1 KB contiguous per instruction, and it issues the loads of two
// entries before consuming them. h never leaves registers: the up dot product
// is reduced across the wave by butterfly and immediately scales the down row.
// [Sparser/Faster/Lighter page (news.neo-ai.one, "Sparser, Faster, Lighter
// Transformer Language Models"), section "TwELL 減掉轉換開銷": one pass computes
// up and down without storing h.]
//
// Work split: workgroup (t, g, s) takes token t, TwELL tiles
// [g*G, (g+1)*G) and every S-th entry of them starting at s; the pack is read
// directly (no prefix over the whole token). Its y contribution is written as
// an fp32 partial row and the partial rows are summed in a fixed order by
// k_ud_reduce (or written straight to y when one workgroup covers the token).
//
// Routed tokens (a tile holding more than E active neurons) go to the dense
// backup [same page, "Hybrid 應對非均勻稀疏"]. With include_routed, this
// kernel evaluates them itself: an overflowing tile is processed densely (its
// T gate values are recomputed, active neurons go through up and down as
// above); at decode token counts that costs less than extra launches, and the
// work is memory-bound either way.
#include "common.cuh"
#include "kernels.cuh"
#include "route.cuh"

namespace ffn {


template <int DT>
struct ElemTraits;
template <>
struct ElemTraits<DT_BF16> {
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  static constexpr int ES = 2;
  __device__ static void to_f32(const uint4 v, float* f) { unpack8(v, f); }
  __device__ static float scalar(const void* p, size_t i) { return bf2f(reinterpret_cast<const uint16_t*>(p)[i]); }
  __device__ static void store(void* p, size_t i, float v) { reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f2bf(v); }
};
template <>
struct ElemTraits<DT_F32> {
  static constexpr int EPC = 4;
  static constexpr int ES = 4;
  __device__ static void to_f32(const uint4 v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static float scalar(const void* p, size_t i) { return reinterpret_cast<const float*>(p)[i]; }
  __device__ static void store(void* p, size_t i, float v) { reinterpret_cast<float*>(p)[i] = v; }
};

__global__ __launch_bounds__(256) void k_route(const RouteDesc r) { route_pass(r); }

hipError_t launch_route(const RouteDesc& r, hipStream_t s) {
  ffn_launch(k_route, dim3(1), dim3(256), 0, s, r);
  return hipGetLastError();
}

// ------------------------------------------------------------------ sparse up + down
template <int DT>
__device__ __forceinline__ float gate_recompute(const UpdownDesc& u, int t, int neuron, const uint4* s_x, int lane,
                                                int nch) {
  using TR = ElemTraits<DT>;
  constexpr int EPC = TR::EPC;
  float s = 0.f;
  if (u.w_gate) {
    const char* row = (const char*)u.w_gate + (size_t)neuron * u.d * TR::ES;
    for (int c = lane; c < nch; c += 64) {
      float f[EPC], xv[EPC];
      TR::to_f32(ldg16(row + (size_t)c * 16), f);
      TR::to_f32(s_x[c], xv);
#pragma unroll
      for (int q = 0; q < EPC; ++q) s = fmaf(f[q], xv[q], s);
    }
  } else {
    const char* row = (const char*)u.u_rows + (size_t)neuron * u.rank * TR::ES;
    const float* tv = u.lr_t + (size_t)t * u.rank;
    const int rch = u.rank / EPC;
    for (int c = lane; c < rch; c += 64) {
      float f[EPC];
      TR::to_f32(ldg16(row + (size_t)c * 16), f);
#pragma unroll
      for (int q = 0; q < EPC; ++q) s = fmaf(f[q], tv[c * EPC + q], s);
    }
  }
  return wave_sum(s);
}

// Entries (and preloaded pack slots) one workgroup holds in LDS.
constexpr int UD_CAP = kUpdownCap;
// phase-B rows in flight per wave
constexpr int UD_BATCH = 16;

// Two phases inside one workgroup (h stays on chip):
//   A  every wave takes entries round-robin: u_i = <W_up[i, :], x_t> over the
//      full row, h_i = a_i u_i into LDS (top-k packs already hold h_i);
//   B  every wave owns a slice of d and accumulates sum_i h_i W_down[i, slice]
//      over all entries of the workgroup. Its first batch of down-row loads
//      does not depend on h, so it is issued before the barrier and overlaps A.
// The workgroup's y contribution leaves as one partial row (no cross-wave
// reduction: the slices are disjoint).
template <int DT, int NW>
__global__ __launch_bounds__(64 * NW) void k_updown(const UpdownDesc u) {
  using TR = ElemTraits<DT>;
  constexpr int EPC = TR::EPC;
  constexpr int CPL = 8;                          // row chunks per lane in phase A (d / EPC <= 512)
  __shared__ uint4 s_x[512];                      // x_t in its storage type, 16-byte chunks
  __shared__ int s_pre[65];                       // entry prefix over the group's tiles
  __shared__ uint8_t s_dense[64];                 // tile overflows: evaluated densely
  __shared__ uint16_t s_idx[UD_CAP];
  __shared__ float s_val[UD_CAP];                 // packed value; then a_i of entry i
  __shared__ int s_nrn[UD_CAP];                   // neuron of entry i (negative: dense candidate)
  __shared__ float s_h[UD_CAP];
  const int d = u.d, T = u.T, E = u.E;
  const int ntiles = u.F / T, nch = d / EPC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = u.tiles_per_group, S = u.slot_split, ngroups = ud_groups(u);
  // the last workgroup (when asked for) only routes the pack, alongside the others
  if (u.route_pass && blockIdx.x == gridDim.x - 1) {
    route_pass(u.route);
    return;
  }
  int bid = blockIdx.x;
  const int s = bid % S;
  bid /= S;
  // token-major: workgroup = token * groups + group; group-major within XCD
  // classes (groups a multiple of 8, one phase): workgroup = ((group / 8) * M +
  // token) * 8 + group % 8, so workgroup b still runs on XCD group % 8 and the
  // workgroups resident together on an XCD share one tile group
  int g, t;
  if (u.xcd_major) {
    const int rest = bid >> 3;
    t = rest % u.M;
    g = (rest / u.M) * 8 + (bid & 7);
  } else {
    g = bid % ngroups;
    t = bid / ngroups;
  }

  // ---- one round of independent loads: tile counts, x_t, the group's slots
  const int j0 = g * G, j1 = min(j0 + G, ntiles), ng = j1 - j0;
  const int32_t* crow = u.cnt + (size_t)t * ntiles;
  int over = 0;
  for (int j = threadIdx.x; j < ntiles; j += blockDim.x) over |= crow[j] > E;
  for (int c = threadIdx.x; c < nch; c += blockDim.x)
    s_x[c] = ldg16((const char*)u.x + ((size_t)t * d + (size_t)c * EPC) * TR::ES);
  {
    const size_t slot0 = ((size_t)t * ntiles + j0) * E;
    for (int q = threadIdx.x; q < ng * E && q < UD_CAP; q += blockDim.x) {
      s_idx[q] = u.idx[slot0 + q];
      s_val[q] = TR::scalar(u.val, slot0 + q);
    }
  }
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int jj = 0; jj < ng; ++jj) {
      s_pre[jj] = acc;
      const int c = crow[j0 + jj];
      s_dense[jj] = c > E ? 1 : 0;
      acc += c > E ? T : c;                      // an overflowing tile is evaluated densely
    }
    s_pre[ng] = min(acc, UD_CAP);
  }
  const bool routed = __syncthreads_or(over) != 0;
  if (routed && !u.include_routed) return;
  const int n_all = s_pre[ng];
  // this workgroup's entries: every S-th starting at s
  const int n = n_all > s ? (n_all - s + S - 1) / S : 0;

  float b = 0.f, cut = 0.f;                       // selection inputs: routed tokens only
  if (routed) {
    b = u.bias ? u.bias[t] : u.bias_scalar;
    cut = (u.sel == SEL_THRESH && u.tau) ? fmaxf(u.tau[t], 0.f) : 0.f;
  }
  // resolve every entry of this workgroup once, in parallel: entry i is slot
  // p = s + i*S of the group; a dense candidate is stored as -(neuron + 1)
  {
    float av[8];
    int nv[8];
    int cnt_here = 0;
    for (int i = threadIdx.x; i < n && cnt_here < 8; i += blockDim.x, ++cnt_here) {
      const int p = s + i * S;
      int jj = 0;
      while (jj + 1 < ng && s_pre[jj + 1] <= p) ++jj;
      const int k = p - s_pre[jj], j = j0 + jj;
      if (s_dense[jj]) {
        nv[cnt_here] = -(j * T + k) - 1;
        av[cnt_here] = 0.f;
      } else {
        nv[cnt_here] = j * T + s_idx[jj * E + k];
        av[cnt_here] = s_val[jj * E + k];
      }
    }
    __syncthreads();                              // s_val is rewritten below
    cnt_here = 0;
    for (int i = threadIdx.x; i < n && cnt_here < 8; i += blockDim.x, ++cnt_here) {
      s_nrn[i] = nv[cnt_here];
      s_val[i] = av[cnt_here];
    }
    __syncthreads();
  }
  auto entry = [&](int i, int& neuron, float& a, bool& dense) {
    const int v = s_nrn[i];
    dense = v < 0;
    neuron = dense ? -v - 1 : v;
    a = s_val[i];
  };

  // phase-B slice of this wave: chunks [wave*cw, wave*cw + cw), one per lane
  const int cw = (nch + NW - 1) / NW;
  const int myc = wave * cw + lane;
  const bool bl = lane < cw && myc < nch;
  const size_t rowb = (size_t)d * TR::ES;

  // ---- phase A (+ the first phase-B batch issued early)
  const bool need_up = !u.down_only;
  uint4 pre[UD_BATCH];
  bool prefetched = false;
  for (int i0 = wave; i0 < n || !prefetched; i0 += 2 * NW) {
    const int i1 = i0 + NW;
    const bool v0 = i0 < n, v1 = i1 < n;
    int n0 = 0, n1 = 0;
    float a0 = 0.f, a1 = 0.f;
    bool d0 = false, d1 = false;
    if (v0) entry(i0, n0, a0, d0);
    if (v1) entry(i1, n1, a1, d1);
    if (v0 && d0) {                               // densely evaluated tile: recompute the gate
      const float z = gate_recompute<DT>(u, t, n0, s_x, lane, nch) + b;
      a0 = z > cut ? z : 0.f;
    }
    if (v1 && d1) {
      const float z = gate_recompute<DT>(u, t, n1, s_x, lane, nch) + b;
      a1 = z > cut ? z : 0.f;
    }
    const bool g0 = v0 && need_up && a0 != 0.f, g1 = v1 && need_up && a1 != 0.f;
    uint4 r0[CPL], r1[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + 64 * c;
      r0[c] = (g0 && ch < nch) ? ldg16((const char*)u.w_up + (size_t)n0 * rowb + (size_t)ch * 16) : uint4{0, 0, 0, 0};
      r1[c] = (g1 && ch < nch) ? ldg16((const char*)u.w_up + (size_t)n1 * rowb + (size_t)ch * 16) : uint4{0, 0, 0, 0};
    }
    if (!prefetched) {                            // first phase-B batch (independent of h)
      int nq[UD_BATCH];
#pragma unroll
      for (int q = 0; q < UD_BATCH; ++q) {
        float aq;
        bool dq;
        nq[q] = 0;
        if (q < n) entry(q, nq[q], aq, dq);
      }
#pragma unroll
      for (int q = 0; q < UD_BATCH; ++q)
        pre[q] = (q < n && bl) ? ldg16((const char*)u.w_down_nm + (size_t)nq[q] * rowb + (size_t)myc * 16) : uint4{0, 0, 0, 0};
      prefetched = true;
    }
    if (v0 || v1) {
      float s0 = 0.f, s1 = 0.f;
      if (need_up) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int ch = lane + 64 * c;
          float f0[EPC], f1[EPC], xv[EPC];
          TR::to_f32(r0[c], f0);
          TR::to_f32(r1[c], f1);
          TR::to_f32(ch < nch ? s_x[ch] : uint4{0, 0, 0, 0}, xv);
#pragma unroll
          for (int q = 0; q < EPC; ++q) {
            s0 = fmaf(f0[q], xv[q], s0);
            s1 = fmaf(f1[q], xv[q], s1);
          }
        }
        s0 = wave_sum(s0);
        s1 = wave_sum(s1);
      }
      if (lane == 0) {
        if (v0) s_h[i0] = need_up ? a0 * s0 : a0;
        if (v1) s_h[i1] = need_up ? a1 * s1 : a1;
      }
    }
  }
  __syncthreads();

  // ---- phase B: this wave's slice of y over every entry
  float ya[EPC];
#pragma unroll
  for (int q = 0; q < EPC; ++q) ya[q] = 0.f;
#pragma unroll
  for (int q = 0; q < UD_BATCH; ++q) {
    if (q < n) {
      const float h = s_h[q];
      float f[EPC];
      TR::to_f32(pre[q], f);
#pragma unroll
      for (int k = 0; k < EPC; ++k) ya[k] = fmaf(h, f[k], ya[k]);
    }
  }
  for (int i0 = UD_BATCH; i0 < n; i0 += UD_BATCH) {
    uint4 rr[UD_BATCH];
    int nq[UD_BATCH];
#pragma unroll
    for (int q = 0; q < UD_BATCH; ++q) {
      float aq;
      bool dq;
      nq[q] = 0;
      if (i0 + q < n) entry(i0 + q, nq[q], aq, dq);
    }
#pragma unroll
    for (int q = 0; q < UD_BATCH; ++q)
      rr[q] = (i0 + q < n && bl) ? ldg16((const char*)u.w_down_nm + (size_t)nq[q] * rowb + (size_t)myc * 16) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < UD_BATCH; ++q) {
      if (i0 + q < n) {
        const float h = s_h[i0 + q];
        float f[EPC];
        TR::to_f32(rr[q], f);
#pragma unroll
        for (int k = 0; k < EPC; ++k) ya[k] = fmaf(h, f[k], ya[k]);
      }
    }
  }
  const int nparts = ngroups * S;
  const size_t part = ((size_t)t * ngroups + g) * S + s;
  if (bl) {
#pragma unroll
    for (int k = 0; k < EPC; ++k) {
      const int e = myc * EPC + k;
      if (nparts == 1) TR::store(u.y, (size_t)t * d + e, ya[k]);
      else u.partial[part * d + e] = ya[k];
    }
  }
}

// y row of token t = ordered sum of its nparts partial rows. Sixteen groups
// of 64 lanes each add every sixteenth partial (8 loads in flight per lane),
// then the groups are combined in order.
constexpr int RED_GROUPS = 16;
template <int DT>
__global__ __launch_bounds__(64 * RED_GROUPS) void k_ud_reduce(const UpdownDesc u) {
  using TR = ElemTraits<DT>;
  __shared__ float s_red[RED_GROUPS][64];
  const int t = blockIdx.y, d = u.d;
  const int e = blockIdx.x * 64 + (threadIdx.x & 63), grp = threadIdx.x >> 6;
  if (!u.include_routed) {
    const int ntiles = u.F / u.T;
    int over = 0;
    for (int j = threadIdx.x; j < ntiles; j += blockDim.x) over |= u.cnt[(size_t)t * ntiles + j] > u.E;
    if (__syncthreads_or(over)) return;
  }
  const int nparts = ud_groups(u) * u.slot_split;
  const float* base = u.partial + (size_t)t * nparts * d + (e < d ? e : 0);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int q = grp;
  for (; q + 7 * RED_GROUPS < nparts; q += 8 * RED_GROUPS) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += base[(size_t)(q + RED_GROUPS * k) * d];
  }
  for (int k = 0; q < nparts; q += RED_GROUPS, ++k) acc[k & 7] += base[(size_t)q * d];
  const float sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  s_red[grp][threadIdx.x & 63] = sum;
  __syncthreads();
  if (grp == 0 && e < d) {
    const int l = threadIdx.x;
    float v = 0.f;
    for (int k = 0; k < RED_GROUPS; ++k) v += s_red[k][l];
    TR::store(u.y, (size_t)t * d + e, v);
  }
}

template <int DT>
static hipError_t go_updown(const UpdownDesc& u, hipStream_t s) {
  dim3 grid(u.M * ud_groups(u) * u.slot_split + (u.route_pass ? 1 : 0));
  if (u.nwaves == 8) ffn_launch((k_updown<DT, 8>), grid, dim3(512), 0, s, u);
  else ffn_launch((k_updown<DT, 4>), grid, dim3(256), 0, s, u);
  return hipGetLastError();
}

hipError_t launch_updown(const UpdownDesc& u, hipStream_t s) {
  if (u.M <= 0) return hipSuccess;
  if (u.tiles_per_group < 1 || u.tiles_per_group > 64 || u.slot_split < 1) return hipErrorInvalidValue;
  if (u.xcd_major && (ud_groups(u) % 8 != 0 || u.slot_split != 1)) return hipErrorInvalidValue;
  const int epc = u.dtype == DT_BF16 ? 8 : 4;
  if (u.d / epc > 512 || (u.d / epc + u.nwaves - 1) / u.nwaves > 64) return hipErrorInvalidValue;
  return u.dtype == DT_BF16 ? go_updown<DT_BF16>(u, s) : go_updown<DT_F32>(u, s);
}

hipError_t launch_updown_reduce(const UpdownDesc& u, hipStream_t s) {
  if (u.M <= 0 || ud_groups(u) * u.slot_split == 1) return hipSuccess;
  dim3 grid((u.d + 63) / 64, u.M);
  if (u.dtype == DT_BF16) ffn_launch(k_ud_reduce<DT_BF16>, grid, dim3(64 * RED_GROUPS), 0, s, u);
  else ffn_launch(k_ud_reduce<DT_F32>, grid, dim3(64 * RED_GROUPS), 0, s, u);
  return hipGetLastError();
}

}  // namespace ffn
