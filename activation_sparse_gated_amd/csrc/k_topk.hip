// WINA top-k selection and TwELL pack, G workgroups per token.
//
// Scores s_i = |h_i| * ||W_down[:, i]||_2 (WINA page, section 3.1) are
// non-negative, so their fp32 bit patterns order like the values. A three-pass
// radix select (11 + 11 + 10 bits, histograms in LDS) finds the exact key of
// the k-th largest score; every key above it is kept, and among keys equal to
// it the lowest indices are kept (prefix count over index order). Thread t
// holds the contiguous run of keys [t C, t C + C) in registers (C <= CW), so
// one block-wide scan (of the counts above and equal to the cut, packed in one
// word) gives every kept neuron its rank in index order. The ranks go to LDS,
// and one wave per TwELL tile writes the tile's slots from them (slot = rank
// minus the kept count before the tile) with coalesced stores. The G
// workgroups of a token each take the selection in full (the same loads and
// passes, so the same cut) and then rank and pack only their own run of
// tiles: the ranking and the pack stores, which bound one workgroup on its
// CU, are spread over G CUs. Optionally the
// kernel also writes the kept neurons as a neuron-ordered list with bf16 h (the
// input of the list-driven down kernel) or h rows with the other neurons
// zeroed (the input of a dense down product).
#include <algorithm>

#include "common.cuh"
#include "kernels.cuh"

namespace ffn {

constexpr int TOPK_THREADS = 1024;

template <int CW, bool HLDS>
__global__ __launch_bounds__(TOPK_THREADS) void k_topk(const TopkDesc d) {
  extern __shared__ uint32_t s_keys[];           // F score bit patterns, then the kept ranks; h (HLDS)
  __shared__ uint32_t s_hist[2][2048];           // radix histograms, alternating by pass
  __shared__ int s_tstart[1024 + 1];             // kept count before each tile (F / T <= 1024)
  __shared__ int s_scan[16];
  __shared__ int s_wtot[2][TOPK_THREADS / 64];   // per-wave histogram sums, alternating by pass
  __shared__ uint32_t s_digit[3], s_above[3];
  const int G = d.G, tok = blockIdx.x / G, wg = blockIdx.x - tok * G, F = d.F, tid = threadIdx.x;
  const int T = d.T, ntiles = F / T;
  const int tlo = wg * ntiles / G, thi = (wg + 1) * ntiles / G;   // this workgroup's tiles
  const int lo = tlo * T, hi = thi * T;
  const float* srow = d.s_buf + (size_t)tok * F;
  float* s_hv = reinterpret_cast<float*>(s_keys + F);
  const float* hrow = d.h_buf + (size_t)tok * F;
  {
    // every load of the thread (scores, and h too) in flight before the first
    // LDS store: one memory round trip
    float sv[CW], hv[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int iu = tid + c * TOPK_THREADS, i = min(iu, F - 1);   // past the end: a re-read, not stored
      sv[c] = srow[i];
      hv[c] = (HLDS && iu >= lo && iu < hi) ? hrow[i] : 0.f;       // h of the own tiles only
    }
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int i = tid + c * TOPK_THREADS;
      if (i < F) {
        s_keys[i] = __float_as_uint(sv[c]);
        if (HLDS && i >= lo && i < hi) s_hv[i] = hv[c];
      }
    }
    for (int i = tid; i < 2048; i += TOPK_THREADS) s_hist[0][i] = 0u;   // the first pass's histogram
  }
  __syncthreads();
  const int C = (F + TOPK_THREADS - 1) / TOPK_THREADS;    // <= CW
  const int i0 = min(F, tid * C), n = min(F, i0 + C) - i0;
  uint32_t key[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) key[c] = c < n ? s_keys[i0 + c] : 0u;

  const int k = min(max(d.k, 0), F);
  uint32_t prefix = 0, pmask = 0;
  int need = k;                                   // elements still to take at the current prefix
  if (k > 0 && k < F) {
    const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
    // three barriers a pass: after the histogram, after the per-wave sums,
    // after the cut digit; the histogram and the sums alternate between two
    // buffers, and the next pass's histogram is cleared while this one is read
    const int lane = tid & 63, wave = tid >> 6;
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = shifts[pass], nb = 1 << widths[pass];
      uint32_t* hist = s_hist[pass & 1];
#pragma unroll
      for (int c = 0; c < CW; ++c)
        if (c < n && (key[c] & pmask) == prefix) atomicAdd(&hist[(key[c] >> sh) & (nb - 1)], 1u);
      __syncthreads();
      // cumulative counts from the largest digit down: thread t owns digits
      // nb-1-2t and nb-2-2t
      const int d0 = nb - 1 - 2 * tid, d1 = d0 - 1;
      const int c0 = d0 >= 0 ? (int)hist[d0] : 0, c1 = d1 >= 0 ? (int)hist[d1] : 0;
      const int incl = wave_incl_scan(c0 + c1);
      if (lane == 63) s_wtot[pass & 1][wave] = incl;
      if (pass < 2)
        for (int i = tid; i < 2048; i += TOPK_THREADS) s_hist[(pass + 1) & 1][i] = 0u;
      __syncthreads();
      int base = 0;
#pragma unroll
      for (int w = 0; w < TOPK_THREADS / 64; ++w)
        if (w < wave) base += s_wtot[pass & 1][w];
      const int ex = base + incl - (c0 + c1);
      if (d0 >= 0 && ex < need && need <= ex + c0) { s_digit[pass] = (uint32_t)d0; s_above[pass] = (uint32_t)ex; }
      if (d1 >= 0 && ex + c0 < need && need <= ex + c0 + c1) { s_digit[pass] = (uint32_t)d1; s_above[pass] = (uint32_t)(ex + c0); }
      __syncthreads();
      prefix |= s_digit[pass] << sh;
      pmask |= (uint32_t)(nb - 1) << sh;
      need -= (int)s_above[pass];
    }
  }

  // selection: a key above tau is kept; among keys equal to tau the first
  // `need` in index order are
  const uint32_t tau = prefix;
  const bool partial = k > 0 && k < F;
  // one scan of the packed pair (keys above tau) << 16 | (keys equal to tau)
  // per run gives both prefixes: the kept count before a run is the keys above
  // tau before it plus min(need, equal keys before it) (both fields < 2^15)
  int ngt = 0, neq = 0;
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    if (c < n && partial) {
      ngt += key[c] > tau ? 1 : 0;
      neq += key[c] == tau ? 1 : 0;
    }
  }
  int tot;
  const int pre2 = block_excl_scan<TOPK_THREADS>((ngt << 16) | neq, s_scan, &tot);
  const int eqb = pre2 & 0xFFFF, gtb = pre2 >> 16;
  int er = eqb;
  uint32_t cm = 0u;                                // kept elements of the run, bit c
  // runs that meet the own tiles: the others need only their prefix
  const bool mine = n > 0 && i0 < hi && i0 + n > lo;
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    if (!mine) break;
    bool sel;
    if (k == 0) sel = false;
    else if (k >= F) sel = true;
    else {
      sel = key[c] > tau;
      if (key[c] == tau) {
        sel = er < need;
        ++er;
      }
    }
    if (c < n && sel) cm |= 1u << c;
  }
  const int pb = k == 0 ? 0 : (k >= F ? i0 : gtb + min(need, eqb));
  const int nsel_tot = k == 0 ? 0 : (k >= F ? F : (tot >> 16) + min(need, tot & 0xFFFF));
  // kept count before each start of an own tile (or of the tile after them)
  // that falls in this run; a start at the run's first element is the prefix
  // itself. The runs that meet the own tiles then overwrite their keys with
  // the kept neurons' ranks (or ~0)
  for (int j = (i0 + T - 1) / T; j * T < i0 + n; ++j)
    if (j >= tlo && j <= thi && (mine || j * T == i0)) s_tstart[j] = pb + __popc(cm & ((1u << (j * T - i0)) - 1u));
  if (tid == 0) s_tstart[ntiles] = nsel_tot;
  if (mine) {
    int p = pb;
#pragma unroll
    for (int c = 0; c < CW; ++c)
      if (c < n) s_keys[i0 + c] = ((cm >> c) & 1u) ? (uint32_t)p++ : ~0u;
  }
  __syncthreads();

  // one wave per tile: its slots (rank within the tile), the list entries and
  // the masked h row, from the ranks in LDS
  const int lane = tid & 63, wave = tid >> 6;
  uint16_t* hm = d.hmask ? reinterpret_cast<uint16_t*>(d.hmask) + (size_t)tok * d.ldhm : nullptr;
  for (int j = tlo + wave; j < thi; j += TOPK_THREADS / 64) {
    const int base = s_tstart[j], cntj = s_tstart[j + 1] - base;
    const size_t slot0 = ((size_t)tok * ntiles + j) * T;   // E == T
    if (lane == 0) d.cnt[(size_t)tok * ntiles + j] = cntj;
#pragma unroll 4
    for (int r = lane; r < T; r += 64) {
      const int i = j * T + r;
      const uint32_t rk = s_keys[i];
      const float hv = HLDS ? s_hv[i] : hrow[i];
      if (rk != ~0u) {
        const size_t slot = slot0 + ((int)rk - base);
        d.idx[slot] = (uint16_t)r;
        if (d.dtype == DT_F32) reinterpret_cast<float*>(d.val)[slot] = hv;
        else reinterpret_cast<uint16_t*>(d.val)[slot] = (uint16_t)f2bf(hv);
        if (d.ul_nrn) {
          d.ul_nrn[rk] = i;
          d.ul_hT[rk] = (uint16_t)f2bf(hv);
        }
      }
      if (hm) hm[i] = rk != ~0u ? (uint16_t)f2bf(hv) : (uint16_t)0;
      if (r >= cntj) {                             // unused slots of the tile
        d.idx[slot0 + r] = 0xFFFF;
        if (d.dtype == DT_F32) reinterpret_cast<float*>(d.val)[slot0 + r] = 0.f;
        else reinterpret_cast<uint16_t*>(d.val)[slot0 + r] = 0;
      }
    }
  }
  if (wg != 0) return;
  if (d.ul_nrn) {
    // list length and the zero pad up to the next multiple of 32
    const int pad = (nsel_tot + 31) / 32 * 32;
    for (int e = nsel_tot + tid; e < pad; e += TOPK_THREADS) {
      d.ul_nrn[e] = 0;
      d.ul_hT[e] = 0;
    }
    if (tid == 0) *d.ul_total = nsel_tot;
  }
  // routing: with E == T no tile can overflow; every token holds exactly k entries
  if (tid == 0) {
    d.route[tok] = 0;
    if (tok == 0) *d.n_dense = 0;
  }
}

hipError_t launch_topk(const TopkDesc& desc, hipStream_t s) {
  if (desc.M <= 0) return hipSuccess;
  TopkDesc d = desc;
  // workgroups per token: up to 16 (and at most one per tile), about one
  // workgroup per CU over all tokens
  const int ntiles = d.T > 0 ? d.F / d.T : 0;
  d.G = std::max(1, std::min({16, ntiles, 256 / d.M}));
  if (d.F > 32 * TOPK_THREADS || d.T <= 0 || d.F % d.T != 0 || d.F / d.T > 1024 || (d.ul_nrn && d.M != 1) ||
      (d.hmask && d.ldhm < d.F))
    return hipErrorInvalidValue;
  // up to 16 keys per thread: h is staged in LDS beside the keys (8 F bytes)
  const bool wide = d.F > 16 * TOPK_THREADS;
  const size_t lds = (size_t)d.F * sizeof(uint32_t) * (wide ? 1 : 2);
  const void* kern = wide ? reinterpret_cast<const void*>(k_topk<32, false>)
                          : reinterpret_cast<const void*>(k_topk<16, true>);
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (wide) ffn_launch(k_topk<32, false>, dim3(d.M * d.G), dim3(TOPK_THREADS), lds, s, d);
  else ffn_launch(k_topk<16, true>, dim3(d.M * d.G), dim3(TOPK_THREADS), lds, s, d);
  return hipGetLastError();
}

}  // namespace ffn
