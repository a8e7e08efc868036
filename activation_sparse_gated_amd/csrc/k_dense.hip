// Dense-side GEMM instantiations (see gemm_core.cuh): the fused gate+up with
// WINA scores, the dense hidden activations, and the output projection.
#include "gemm_core.cuh"

namespace ffn {

hipError_t launch_gemm_dense(const GemmDesc& g, const EpiDesc& e, hipStream_t s) {
  const dim3 grid = gemm_grid(g);
  if (g.dtype == DT_F32) {
    if (g.mt != 16) return hipErrorInvalidValue;
    switch (e.kind) {
      case EPI_WINA: return go_f32<2, EPI_WINA>(g, e, grid, s);
      case EPI_DENSE_H: return g.nmat == 2 ? go_f32<2, EPI_DENSE_H>(g, e, grid, s) : go_f32<1, EPI_DENSE_H>(g, e, grid, s);
      case EPI_Y: return go_f32<1, EPI_Y>(g, e, grid, s);
    }
    return hipErrorInvalidValue;
  }
  if (g.gemv) {
    switch (e.kind) {
      case EPI_WINA: return go_gemv<2, EPI_WINA>(g, e, grid, s);
      case EPI_DENSE_H: return g.nmat == 2 ? go_gemv<2, EPI_DENSE_H>(g, e, grid, s) : go_gemv<1, EPI_DENSE_H>(g, e, grid, s);
      case EPI_Y: return go_gemv<1, EPI_Y>(g, e, grid, s);
    }
    return hipErrorInvalidValue;
  }
  if (g.bmode != B_NATIVE) return hipErrorInvalidValue;
  switch (e.kind) {
    case EPI_WINA: return pick_shape<B_NATIVE, 2, EPI_WINA>(g, e, grid, s);
    case EPI_DENSE_H:
      return g.nmat == 2 ? pick_shape<B_NATIVE, 2, EPI_DENSE_H>(g, e, grid, s) : pick_shape<B_NATIVE, 1, EPI_DENSE_H>(g, e, grid, s);
    case EPI_Y: return pick_shape<B_NATIVE, 1, EPI_Y>(g, e, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ffn
