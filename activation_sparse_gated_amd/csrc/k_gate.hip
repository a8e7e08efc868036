// Gate-side GEMM instantiations: fp32 stores (low-rank first stage, gate
// values) and the TwELL-emitting gate (see gemm_core.cuh), plus the launch
// dispatcher for every GEMM epilogue.
#include "gemm_core.cuh"

namespace ffn {

constexpr int kSkPreferMaxM = 256;

hipError_t launch_gemm_pack(const GemmDesc& g, const EpiDesc& e, hipStream_t s) {
  const dim3 grid = gemm_grid(g);
  if (g.dtype == DT_F32) {
    if (g.mt != 16) return hipErrorInvalidValue;
    return e.kind == EPI_TWELL ? go_f32<1, EPI_TWELL>(g, e, grid, s) : go_f32<1, EPI_STORE_F32>(g, e, grid, s);
  }
  if (g.gemv) return e.kind == EPI_TWELL ? go_gemv<1, EPI_TWELL>(g, e, grid, s) : go_gemv<1, EPI_STORE_F32>(g, e, grid, s);
  const bool split = g.bmode == B_F32_SPLIT;
  if (e.kind == EPI_TWELL)
    return split ? pick_shape<B_F32_SPLIT, 1, EPI_TWELL>(g, e, grid, s) : pick_shape<B_NATIVE, 1, EPI_TWELL>(g, e, grid, s);
  return split ? pick_shape<B_F32_SPLIT, 1, EPI_STORE_F32>(g, e, grid, s)
               : pick_shape<B_NATIVE, 1, EPI_STORE_F32>(g, e, grid, s);
}

hipError_t launch_gemm(const GemmDesc& g, const EpiDesc& e, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  // up to 256 tokens the skinny kernel's 64-token blocks beat the 128 x 128
  // prefill tiles, which leave most CUs idle there (LoPA shape, dense FFN: 128
  // tokens 371 -> 166 us, 256 tokens 377 -> 293 us; at 512 tokens 407 vs
  // 526 us); the TwELL gate keeps the prefill kernel's epilogue
  const bool sk_first = g.M <= kSkPreferMaxM && e.kind != EPI_TWELL && sk_ok(g, e);
  if (pf_ok(g, e) && !g.no_pf && !sk_first) return launch_gemm_pf(g, e, s);
  if (sk_ok(g, e)) return launch_gemm_sk(g, e, s);
  if (g.nwaves != 4 && g.nwaves != 16) return hipErrorInvalidValue;
  if (e.kind == EPI_STORE_F32 || e.kind == EPI_TWELL) return launch_gemm_pack(g, e, s);
  return launch_gemm_dense(g, e, s);
}

}  // namespace ffn
