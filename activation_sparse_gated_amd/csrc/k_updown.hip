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

namespace ffn {

constexpr int UD_WAVES = 4;

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

// ------------------------------------------------------------------ routing
// One workgroup (256 threads): route_t = any tile with cnt > E; dense_list =
// routed ids ascending; n_dense. Then advances the look-back epoch (the gate
// pass that wrote this pack has completed).
__device__ void route_pass(const RouteDesc& r) {
  __shared__ int s_over[1024];
  __shared__ int s_scan[4];
  int base = 0;
  for (int c0 = 0; c0 < r.M; c0 += 1024) {
    const int n = min(1024, r.M - c0);
    for (int i = threadIdx.x; i < 1024; i += blockDim.x) s_over[i] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < n * r.ntiles; p += blockDim.x) {
      const int t = p / r.ntiles;
      if (r.cnt[(size_t)(c0 + t) * r.ntiles + (p % r.ntiles)] > r.E) s_over[t] = 1;
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

__global__ __launch_bounds__(256) void k_route(const RouteDesc r) { route_pass(r); }

hipError_t launch_route(const RouteDesc& r, hipStream_t s) {
  hipLaunchKernelGGL(k_route, dim3(1), dim3(256), 0, s, r);
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

// Preloaded pack slots per workgroup (idx + value), when the group is small.
constexpr int UD_PRELOAD = 2048;

template <int CPL, int DT, int NW>
__global__ __launch_bounds__(64 * NW) void k_updown(const UpdownDesc u) {
  using TR = ElemTraits<DT>;
  constexpr int EPC = TR::EPC;
  constexpr int VPL = CPL * EPC;                  // values per lane
  constexpr int HALF = NW > 4 ? NW / 2 : NW;      // waves whose partial rows live in LDS
  __shared__ float s_y[HALF][CPL * 64 * EPC];
  __shared__ uint4 s_x[CPL * 64];                 // x_t in its storage type, 16-byte chunks
  __shared__ int s_lim[64];                       // entries per tile of the group
  __shared__ uint16_t s_idx[UD_PRELOAD];
  __shared__ float s_val[UD_PRELOAD];
  const int d = u.d, T = u.T, E = u.E;
  const int ntiles = u.F / T, nch = d / EPC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = u.tiles_per_group, S = u.slot_split, ngroups = ud_groups(u);
  int bid = blockIdx.x;
  const int s = bid % S;
  bid /= S;
  const int g = bid % ngroups, t = bid / ngroups;
  if (u.route_pass && blockIdx.x == 0) route_pass(u.route);

  // one round of independent loads: the token's tile counts (routing test),
  // x_t, and this group's pack slots
  const int j0 = g * G, j1 = min(j0 + G, ntiles), ng = j1 - j0;
  const int32_t* crow = u.cnt + (size_t)t * ntiles;
  int over = 0;
  for (int j = threadIdx.x; j < ntiles; j += blockDim.x) over |= crow[j] > E;
  for (int c = threadIdx.x; c < nch; c += blockDim.x)
    s_x[c] = ldg16((const char*)u.x + ((size_t)t * d + (size_t)c * EPC) * TR::ES);
  const bool preload = ng * E <= UD_PRELOAD;
  if (preload) {
    const size_t slot0 = ((size_t)t * ntiles + j0) * E;
    for (int q = threadIdx.x; q < ng * E; q += blockDim.x) {
      s_idx[q] = u.idx[slot0 + q];
      s_val[q] = TR::scalar(u.val, slot0 + q);
    }
  }
  for (int jj = threadIdx.x; jj < ng; jj += blockDim.x) {
    const int c = crow[j0 + jj];
    s_lim[jj] = c > E ? T : c;                    // an overflowing tile is evaluated densely
  }
  const bool routed = __syncthreads_or(over) != 0;
  if (routed && !u.include_routed) return;

  // selection inputs are read only for a routed token evaluated here (the
  // standalone sparse pass passes no bias / threshold pointers)
  float b = 0.f, cut = 0.f;
  if (routed) {
    b = u.bias ? u.bias[t] : u.bias_scalar;
    cut = (u.sel == SEL_THRESH && u.tau) ? fmaxf(u.tau[t], 0.f) : 0.f;
  }
  float ya[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) ya[q] = 0.f;

  // this wave's candidates: slots k = s + S*wave + S*NW*i of every tile of the
  // group, valid while k < s_lim (ascending tile, then slot)
  const int kfirst = s + S * wave, kstep = S * NW;
  int cj = 0, ck = kfirst;
  auto next = [&](int& j, int& k) -> bool {
    while (cj < ng && ck >= s_lim[cj]) {
      ++cj;
      ck = kfirst;
    }
    if (cj >= ng) return false;
    j = cj;
    k = ck;
    ck += kstep;
    return true;
  };
  auto entry = [&](int jj, int k, int& neuron, float& a, bool& dense) {
    const int j = j0 + jj;
    dense = crow[j] > E;
    if (dense) {
      neuron = j * T + k;
      a = 0.f;
    } else if (preload) {
      neuron = j * T + s_idx[jj * E + k];
      a = s_val[jj * E + k];
    } else {
      const size_t ent = ((size_t)t * ntiles + j) * E + k;
      neuron = j * T + u.idx[ent];
      a = TR::scalar(u.val, ent);
    }
  };

  const bool need_up = !u.down_only;
  // 4-wave workgroups keep two entries' rows in flight per wave, 8-wave ones
  // one (same bytes in flight per CU, half the registers)
  constexpr bool PAIR = NW <= 4;
  int ja, ka, jb = 0, kb = 0;
  while (next(ja, ka)) {
    const bool has2 = PAIR && next(jb, kb);
    int n1, n2 = 0;
    float a1, a2 = 0.f;
    bool d1, d2 = false;
    entry(ja, ka, n1, a1, d1);
    if (has2) entry(jb, kb, n2, a2, d2);
    if (d1) {                                      // densely evaluated tile: recompute the gate
      const float z = gate_recompute<DT>(u, t, n1, s_x, lane, nch) + b;
      a1 = z > cut ? z : 0.f;
    }
    if (has2 && d2) {
      const float z = gate_recompute<DT>(u, t, n2, s_x, lane, nch) + b;
      a2 = z > cut ? z : 0.f;
    }
    const bool go1 = a1 != 0.f || !d1, go2 = has2 && (a2 != 0.f || !d2);
    const char* up1 = (const char*)u.w_up + (size_t)n1 * d * TR::ES;
    const char* dn1 = (const char*)u.w_down_nm + (size_t)n1 * d * TR::ES;
    const char* up2 = (const char*)u.w_up + (size_t)n2 * d * TR::ES;
    const char* dn2 = (const char*)u.w_down_nm + (size_t)n2 * d * TR::ES;
    constexpr int C2 = PAIR ? CPL : 1;
    uint4 ur1[CPL], dr1[CPL], ur2[C2], dr2[C2];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < nch;
      ur1[i] = (ok && go1 && need_up) ? ldg16(up1 + (size_t)c * 16) : uint4{0, 0, 0, 0};
      dr1[i] = (ok && go1) ? ldg16(dn1 + (size_t)c * 16) : uint4{0, 0, 0, 0};
      if (PAIR) {
        ur2[i % C2] = (ok && go2 && need_up) ? ldg16(up2 + (size_t)c * 16) : uint4{0, 0, 0, 0};
        dr2[i % C2] = (ok && go2) ? ldg16(dn2 + (size_t)c * 16) : uint4{0, 0, 0, 0};
      }
    }
    float h1 = a1, h2 = a2;
    if (need_up) {
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        float f1[EPC], f2[EPC], xv[EPC];
        TR::to_f32(ur1[i], f1);
        TR::to_f32(PAIR ? ur2[i % C2] : uint4{0, 0, 0, 0}, f2);
        TR::to_f32(c < nch ? s_x[c] : uint4{0, 0, 0, 0}, xv);
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          s1 = fmaf(f1[q], xv[q], s1);
          s2 = fmaf(f2[q], xv[q], s2);
        }
      }
      h1 = a1 * wave_sum(s1);
      h2 = a2 * wave_sum(s2);
    }
    if (!go1) h1 = 0.f;
    if (!go2) h2 = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      float f1[EPC], f2[EPC];
      TR::to_f32(dr1[i], f1);
      TR::to_f32(PAIR ? dr2[i % C2] : uint4{0, 0, 0, 0}, f2);
#pragma unroll
      for (int q = 0; q < EPC; ++q)
        ya[i * EPC + q] = PAIR ? fmaf(h2, f2[q], fmaf(h1, f1[q], ya[i * EPC + q])) : fmaf(h1, f1[q], ya[i * EPC + q]);
    }
    if (PAIR && !has2) break;
  }

  // combine the waves in a fixed order: the first HALF store, the rest add
  // into the same rows, then the rows are summed
  if (wave < HALF) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int q = 0; q < EPC; ++q) s_y[wave][(i * 64 + lane) * EPC + q] = ya[i * EPC + q];
  }
  __syncthreads();
  if (NW > HALF && wave >= HALF) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int q = 0; q < EPC; ++q) s_y[wave - HALF][(i * 64 + lane) * EPC + q] += ya[i * EPC + q];
  }
  if (NW > HALF) __syncthreads();
  const int nparts = ngroups * S;
  const size_t part = ((size_t)t * ngroups + g) * S + s;
  for (int e = threadIdx.x; e < d; e += blockDim.x) {
    float v = s_y[0][e];
#pragma unroll
    for (int w = 1; w < HALF; ++w) v += s_y[w][e];
    if (nparts == 1) TR::store(u.y, (size_t)t * d + e, v);
    else u.partial[part * d + e] = v;
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

template <int DT, int NW>
static hipError_t go_updown_nw(const UpdownDesc& u, hipStream_t s) {
  const int epc = DT == DT_BF16 ? 8 : 4;
  const int cpl = (u.d / epc + 63) / 64;
  dim3 grid(u.M * ud_groups(u) * u.slot_split), blk(64 * NW);
  switch (cpl) {
    case 1: hipLaunchKernelGGL((k_updown<1, DT, NW>), grid, blk, 0, s, u); break;
    case 2: hipLaunchKernelGGL((k_updown<2, DT, NW>), grid, blk, 0, s, u); break;
    case 3:
    case 4: hipLaunchKernelGGL((k_updown<4, DT, NW>), grid, blk, 0, s, u); break;
    case 5: case 6: case 7:
    case 8: hipLaunchKernelGGL((k_updown<8, DT, NW>), grid, blk, 0, s, u); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
static hipError_t go_updown(const UpdownDesc& u, hipStream_t s) {
  return u.nwaves == 8 ? go_updown_nw<DT, 8>(u, s) : go_updown_nw<DT, 4>(u, s);
}

hipError_t launch_updown(const UpdownDesc& u, hipStream_t s) {
  if (u.M <= 0) return hipSuccess;
  if (u.tiles_per_group < 1 || u.tiles_per_group > 64 || u.slot_split < 1) return hipErrorInvalidValue;
  return u.dtype == DT_BF16 ? go_updown<DT_BF16>(u, s) : go_updown<DT_F32>(u, s);
}

hipError_t launch_updown_reduce(const UpdownDesc& u, hipStream_t s) {
  if (u.M <= 0 || ud_groups(u) * u.slot_split == 1) return hipSuccess;
  dim3 grid((u.d + 63) / 64, u.M);
  if (u.dtype == DT_BF16) hipLaunchKernelGGL(k_ud_reduce<DT_BF16>, grid, dim3(64 * RED_GROUPS), 0, s, u);
  else hipLaunchKernelGGL(k_ud_reduce<DT_F32>, grid, dim3(64 * RED_GROUPS), 0, s, u);
  return hipGetLastError();
}

}  // namespace ffn
