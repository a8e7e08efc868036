// WINA top-k selection and TwELL pack, one workgroup per token.
//
// Scores s_i = |h_i| * ||W_down[:, i]||_2 (WINA page, section 3.1) are
// non-negative, so their fp32 bit patterns order like the values. A three-pass
// radix select (11 + 11 + 10 bits, histograms in LDS) finds the exact key of
// the k-th largest score; every key above it is kept, and among keys equal to
// it the lowest indices are kept (prefix count over index order). The kept
// neurons are then written per tile in ascending order with their h values.
#include "common.cuh"
#include "kernels.cuh"

namespace ffn {

constexpr int TOPK_THREADS = 1024;

__global__ __launch_bounds__(TOPK_THREADS) void k_topk(const TopkDesc d) {
  extern __shared__ uint32_t s_keys[];           // F score bit patterns
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_selbits[1024];           // F / 32 selection bits (F <= 32768)
  __shared__ int s_scan[16];
  __shared__ uint32_t s_digit, s_above;
  const int tok = blockIdx.x, F = d.F, tid = threadIdx.x;
  const float* srow = d.s_buf + (size_t)tok * F;
  for (int i = tid; i < F; i += TOPK_THREADS) s_keys[i] = __float_as_uint(srow[i]);
  for (int i = tid; i < (F + 31) / 32; i += TOPK_THREADS) s_selbits[i] = 0u;
  __syncthreads();

  const int k = min(max(d.k, 0), F);
  uint32_t prefix = 0, pmask = 0;
  int need = k;                                   // elements still to take at the current prefix
  if (k > 0 && k < F) {
    const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = shifts[pass], nb = 1 << widths[pass];
      for (int i = tid; i < 2048; i += TOPK_THREADS) s_hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < F; i += TOPK_THREADS) {
        const uint32_t key = s_keys[i];
        if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      // cumulative counts from the largest digit down: thread t owns digits
      // nb-1-2t and nb-2-2t
      const int d0 = nb - 1 - 2 * tid, d1 = d0 - 1;
      const int c0 = d0 >= 0 ? (int)s_hist[d0] : 0, c1 = d1 >= 0 ? (int)s_hist[d1] : 0;
      int total;
      const int ex = block_excl_scan<TOPK_THREADS>(c0 + c1, s_scan, &total);
      if (d0 >= 0 && ex < need && need <= ex + c0) { s_digit = (uint32_t)d0; s_above = (uint32_t)ex; }
      if (d1 >= 0 && ex + c0 < need && need <= ex + c0 + c1) { s_digit = (uint32_t)d1; s_above = (uint32_t)(ex + c0); }
      __syncthreads();
      prefix |= s_digit << sh;
      pmask |= (uint32_t)(nb - 1) << sh;
      need -= (int)s_above;
      __syncthreads();
    }
  }
  // selection bits: key > tau, or key == tau among the first `need` in index order
  const uint32_t tau = prefix;
  int base = 0;
  for (int c0 = 0; c0 < F; c0 += TOPK_THREADS) {
    const int i = c0 + tid;
    const uint32_t key = i < F ? s_keys[i] : 0u;
    const int eq = (i < F && k > 0 && k < F && key == tau) ? 1 : 0;
    int tot;
    const int r = block_excl_scan<TOPK_THREADS>(eq, s_scan, &tot);
    bool sel;
    if (k == 0) sel = false;
    else if (k >= F) sel = i < F;
    else sel = i < F && (key > tau || (eq && base + r < need));
    if (sel) atomicOr(&s_selbits[i >> 5], 1u << (i & 31));
    base += tot;
  }
  __syncthreads();

  // pack: one wave per tile, 64 columns per ballot
  const int ntiles = F / d.T, lane = tid & 63, wave = tid >> 6;
  const float* hrow = d.h_buf + (size_t)tok * F;
  for (int j = wave; j < ntiles; j += TOPK_THREADS / 64) {
    const size_t slot0 = ((size_t)tok * ntiles + j) * d.T;  // E == T
    int run = 0;
    for (int c = 0; c < d.T; c += 64) {
      const int r = c + lane;
      const int i = j * d.T + r;
      const bool sel = r < d.T && ((s_selbits[i >> 5] >> (i & 31)) & 1u);
      const uint64_t bal = ballot64(sel);
      const int pos = run + __popcll(bal & lanemask_lt());
      if (sel) {
        d.idx[slot0 + pos] = (uint16_t)r;
        if (d.dtype == DT_F32) reinterpret_cast<float*>(d.val)[slot0 + pos] = hrow[i];
        else reinterpret_cast<uint16_t*>(d.val)[slot0 + pos] = (uint16_t)f2bf(hrow[i]);
      }
      run += __popcll(bal);
    }
    if (lane == 0) d.cnt[(size_t)tok * ntiles + j] = run;
    for (int s = run + lane; s < d.T; s += 64) {
      d.idx[slot0 + s] = 0xFFFF;
      if (d.dtype == DT_F32) reinterpret_cast<float*>(d.val)[slot0 + s] = 0.f;
      else reinterpret_cast<uint16_t*>(d.val)[slot0 + s] = 0;
    }
  }
  // routing: with E == T no tile can overflow; every token holds exactly k entries
  if (tid == 0) {
    d.route[tok] = 0;
    if (tok == 0) *d.n_dense = 0;
  }
}

hipError_t launch_topk(const TopkDesc& d, hipStream_t s) {
  if (d.M <= 0) return hipSuccess;
  const size_t lds = (size_t)d.F * sizeof(uint32_t);
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  ffn_launch(k_topk, dim3(d.M), dim3(TOPK_THREADS), lds, s, d);
  return hipGetLastError();
}

}  // namespace ffn
