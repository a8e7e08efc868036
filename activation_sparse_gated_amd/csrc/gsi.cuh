// Internal interface of the gated subspace (GSI) linear map: descriptors and
// launches shared by the C ABI layer (gsi_api.hip) and the kernels (k_gsi.hip).
#pragma once
#include "kernels.cuh"

namespace ffn {

constexpr int kGsiMaxM = 16;        // tokens per launch group
constexpr int kGsiProjMaxNpl = 4;   // 512-element chunks a lane loads per item (d_in <= 16384)
constexpr int kGsiMaxNl = 8;        // k-rows a lane holds in flight
constexpr int kGsiMaxK = 512;       // largest rank
constexpr int kGsiResWaves = 8;     // waves of a residual workgroup
constexpr int kGsiResParts = 64;    // residual workgroups the plan aims for at most
constexpr int kGsiResRowsMax = 512;  // rows of a residual workgroup at most (x of its rows staged in LDS)

struct GsiDesc {
  int d, dout, k, M;            // input width, output width, rank, tokens of this group (1..16)
  const uint16_t* w;            // [dout x d]
  const uint16_t* vk;           // [d x k]
  const uint16_t* vt;           // [k x d]
  const uint16_t* img;          // [dout x k]
  const uint16_t* x;            // the group's first token row of x [M x d]
  uint16_t* y;                  // the group's first row of y [M x dout]
  float* g;                     // [16 x k] projections of the group
  float* part;                  // [2 x 16 x nres]: ||r||^2 parts, then ||x||^2 parts
  int32_t* counter;             // slow tokens of the earlier groups of this call
  float eps;
  int force_slow;               // every token takes W x (the dense baseline)
  int tok0;                     // index of the group's first token within the call
  float* rho;                   // [m] or null (whole call)
  int32_t* slow_list;           // [m] or null
  int32_t* n_slow;              // or null
  // launch shapes (gsi_plan)
  int proj_ipr, proj_npl, proj_rpb;   // items per V_k^T row, chunks per item, rows per workgroup
  int lpr;                            // lanes per k-row (power of two, 8 elements each)
  int res_nl, nres;                   // k-rows per lane and workgroups of the residual kernel
  int out_nl, nout;                   // the same for the output kernel
  int lpr4, out_nl4, nout4;           // the output kernel with several tokens: 4 chunks a lane
};

bool gsi_plan(GsiDesc& d, int cus);
// Most residual workgroups any plan gives for this shape (parts the workspace holds).
int gsi_max_parts(int d_in, int k);
hipError_t launch_gsi_proj(const GsiDesc& d, hipStream_t s);
hipError_t launch_gsi_resid(const GsiDesc& d, hipStream_t s);
hipError_t launch_gsi_out(const GsiDesc& d, hipStream_t s);
// img[o][c] = bf16(sum_j w[o][j] * vt[c][j]), fp32 accumulation in j order.
hipError_t launch_gsi_image(const uint16_t* w, const uint16_t* vt, uint16_t* img, int dout, int d, int k,
                            hipStream_t s);

}  // namespace ffn
