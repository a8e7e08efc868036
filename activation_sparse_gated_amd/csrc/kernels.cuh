// Internal interface between the C ABI layer and the kernel translation units.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffn {

// Events the next kernel launched through ffn_launch on this host thread
// records from its own dispatch (its start and end timestamps, as a profiler
// sees them); cleared once used. Set by the per-kernel timing of the C ABI.
struct LaunchEvents {
  hipEvent_t start, stop;
};
extern thread_local LaunchEvents tl_launch_events;

// Every kernel of the library is launched here.
template <typename F, typename... Args>
inline void ffn_launch(F kernel, const dim3& grid, const dim3& block, size_t lds, hipStream_t s, Args... args) {
  const LaunchEvents ev = tl_launch_events;
  tl_launch_events = LaunchEvents{nullptr, nullptr};
  hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0u, args...);
}

enum Dtype : int { DT_F32 = 0, DT_BF16 = 1 };
enum Act : int { ACT_RELU = 0, ACT_SILU = 1 };
enum Sel : int { SEL_BIAS = 0, SEL_THRESH = 1, SEL_TOPK = 2 };
enum BMode : int { B_NATIVE = 0, B_F32_SPLIT = 1 };
enum EpiKind : int { EPI_STORE_F32 = 0, EPI_TWELL = 1, EPI_WINA = 2, EPI_DENSE_H = 3, EPI_Y = 4 };

// C[n, m] = sum_k A[n, k] * B[m, k]: A holds weight rows (one or two matrices
// stacked per tile), B holds token rows. Both are K-contiguous.
struct GemmDesc {
  int dtype;              // element type of A (and of B unless bmode = B_F32_SPLIT)
  const void* A0;         // rows [0, nrows) of matrix 0
  const void* A1;         // matrix 1 (nmat == 2): the second half of every tile
  int nmat;               // 1 or 2
  int nrows;              // rows per matrix
  int lda;                // elements
  int K;                  // contraction length (multiple of 32)
  const void* B;          // token rows
  int ldb;                // elements
  int bmode;              // B_NATIVE or B_F32_SPLIT (fp32 B split into bf16 hi + lo)
  int b_nsum;             // B is the sum of b_nsum fp32 slabs (B_F32_SPLIT / fp32), >= 1
  long long b_slab;       // elements between consecutive B slabs
  int M;                  // token count bound known on the host
  const int32_t* gather;  // B row of token slot m is gather[m]; null = m
  const int32_t* m_dev;   // device-side token count (dense backup); null = M
  int nt;                 // rows per workgroup tile (16, 32, 64, 128; per matrix * nmat)
  int mt;                 // tokens per workgroup (16, 32 or 64)
  int nwaves;             // waves per workgroup (4 or 16)
  int gemv;               // decode GEMV (VALU) instead of MFMA tiles (bf16, M <= 8)
  int ks;                 // workgroups splitting K; each writes its own output slab (>= 1)
  uint32_t* ctrl;         // control block (epoch of the look-back words, wait limits, error word)
  int no_pf;              // 1: never the prefill-shaped kernel (tuning switch)
  // prefill-shaped kernel with ks > 1 (output rows y, device-side token count):
  // slice z of K writes fp32 partials kpart[(z * kpart_m + m) * nrows + n]
  float* kpart;
  int kpart_m;
  // skinny kernel (9..127 tokens, output rows y): K may be split over
  // workgroups whose fp32 partial slabs [ks x M x nrows] go here, at most
  // skpart_rows = ks * M rows; null: no K split
  float* skpart;
  int skpart_rows;
};

struct EpiDesc {
  int kind;               // EpiKind
  int F;                  // neurons (rows per matrix)
  int out_f32;            // outputs in fp32 (fp32 configs) instead of bf16
  const int32_t* tok_of;  // token id of slot m (dense backup); null = m
  const float* bias;      // [tokens] or null
  float bias_scalar;
  const float* tau;       // [tokens] (THRESH)
  int sel, act;
  float* g_debug;         // [tokens x F] gate before bias
  float* s_debug;         // [tokens x F] WINA scores
  // EPI_STORE_F32: out + ksi * out_slab + m * ldo + n
  float* out; int ldo; long long out_slab;
  float* t_out;           // EPI_TWELL on the low-rank gate: tile 0 stores the summed t here
  // EPI_TWELL
  int T, E;
  int32_t* cnt; uint16_t* idx; void* val;
  uint64_t* lb;           // look-back words [F / nt sub-tiles x lb_ld tokens] (sub-tiled TwELL tiles)
  int lb_ld;              // token stride of lb (>= the token count)
  // EPI_WINA
  const float* colnorm; float* s_buf; float* h_buf;
  // EPI_DENSE_H
  void* hout; int ldh; const float* g_ext;
  // EPI_Y
  void* y; int ldy; const int32_t* yrows;
};

hipError_t launch_gemm(const GemmDesc& g, const EpiDesc& e, hipStream_t s);
// y [m x ldy] = A [nrows x K] x for m tokens (bf16) with the dense GEMM kernels.
hipError_t dense_rows_bf16(const void* A, int nrows, int K, const void* x, int m, void* y, int ldy, int cus,
                           hipStream_t s);

// Transpose rows x cols (row-major) -> cols x rows, element size 2 or 4 bytes.
hipError_t launch_transpose(const void* src, void* dst, int rows, int cols, int esize, hipStream_t s);
hipError_t launch_transpose_ld(const void* src, void* dst, int rows, int cols, int ldd, int esize, hipStream_t s);
// c[i] = || row i of the neuron-major matrix [F x d] ||_2 (fp32, correctly rounded sqrt).
hipError_t launch_rownorm(const void* w, float* c, int F, int d, int dtype, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s);
// slab 0 += slabs 1..nslabs-1 (in order), n floats each, slab stride `stride`.
hipError_t launch_slab_sum(float* slabs, int nslabs, size_t stride, size_t n, hipStream_t s);

struct TopkDesc {
  int M, F, k, T, dtype;
  const float* s_buf; const float* h_buf;
  int32_t* cnt; uint16_t* idx; void* val;
  uint8_t* route; int32_t* dense_list; int32_t* n_dense;
  // optional outputs (null: not written)
  int32_t* ul_nrn; uint16_t* ul_hT; int32_t* ul_total;   // one token: kept neurons ascending, bf16 h, count
  void* hmask; int ldhm;                                  // bf16 h rows, unselected neurons zero
  int G;                                                  // workgroups per token (set by the launcher)
};
hipError_t launch_topk(const TopkDesc& d, hipStream_t s);

// Routing of a TwELL pack: route_t = any tile with cnt > E, dense_list = the
// routed ids ascending, n_dense; also advances the look-back epoch.
struct RouteDesc {
  int M, ntiles, E;
  const int32_t* cnt;
  uint8_t* route; int32_t* dense_list; int32_t* n_dense;
  uint32_t* ctrl;
};
hipError_t launch_route(const RouteDesc& r, hipStream_t s);

// TwELL pack of m tokens from their gate values g [m x F] (fp32, before the
// bias), one wave per (token, TwELL tile): the selection z = g + b > cut of
// the other epilogues, the first min(cnt, E) active offsets ascending, values
// rounded to the pack type, padding, and the true count.
struct PackGDesc {
  int M, F, T, E, sel, out_f32;
  const float* g;
  const float* bias; float bias_scalar; const float* tau;
  int32_t* cnt; uint16_t* idx; void* val;
};
hipError_t launch_pack_g(const PackGDesc& d, hipStream_t s);

struct UpdownDesc {
  int dtype, M, d, F, T, E;
  int down_only;          // TOPK: pack values are h, no up product
  const void* x; const void* w_up; const void* w_down_nm;
  const int32_t* cnt; const uint16_t* idx; const void* val;
  void* y;
  float* partial;         // [M x ngroups x slot_split x d]
  int tiles_per_group;    // G: tiles handled by one workgroup
  int slot_split;         // S: workgroups sharing one tile group (entry phase)
  int nwaves;             // waves per workgroup (4 or 8)
  int xcd_major;          // 1: workgroups dealt group-major within each XCD class (groups % 8 == 0, S == 1)
  int route_pass;         // block 0 also routes the pack (route / dense_list / n_dense, epoch)
  RouteDesc route;
  int include_routed;     // evaluate routed tokens here: overflowing tiles densely
  // gate recompute for routed tokens
  const void* w_gate;     // full gate rows [F x d], or null for the low-rank gate
  const void* u_rows;     // low-rank U [F x rank]
  const float* lr_t;      // low-rank intermediate t [M x rank] (fp32)
  int rank;
  const float* bias; float bias_scalar; const float* tau; int sel;
};
// Input-side selection of the gate projection (k_input.hip), bf16.
struct InDesc {
  int M, d, k, N, groups;       // tokens, input channels, kept per token, gate outputs (F or rank), channel groups
  const void* x;                // [M x d] bf16
  const float* colnorm;         // [d] ||W[:, j]||_2
  int32_t* kidx;                // [M x k] kept channels, ascending
  uint16_t* kval;               // [M x k] their x values (bf16)
  const uint16_t* wt;           // W^T [d x N], input-major
  float* part;                  // [groups x M x N] partial sums over the channel groups
  // k_in_pack (full gate): selection and TwELL pack from the summed partials
  int T, E, sel;
  const float* bias; float bias_scalar; const float* tau;
  int32_t* cnt; uint16_t* idx; void* val; float* g_debug;
};
int in_groups(int N, int k);
bool in_ok(const InDesc& d);
hipError_t launch_in_select(const InDesc& d, hipStream_t s);
hipError_t launch_in_gemv(const InDesc& d, hipStream_t s);
hipError_t launch_in_sum(const InDesc& d, hipStream_t s);
hipError_t launch_in_pack(const InDesc& d, hipStream_t s);

// One-token dense weight streams (k_sgemv.hip), bf16, m = 1: rows of A
// dotted with a vector, optionally with a gate matrix per row.
enum SgEpi : int {
  SG_OUT = 0,    // out[row] fp32
  SG_Y = 1,      // y[row], bf16 or fp32
  SG_HID = 2,    // hout[row] = bf16(a(g + b) * u), the selection's mask applied
  SG_SCORE = 3   // WINA: h = a(g + b) u, s = |h| c into h_buf / s_buf
};
struct Sgemv1Desc {
  int N, K, Kg;                 // rows; contraction of A; contraction of the gate rows
  const uint16_t* A;            // [N x K] bf16 (u rows for SG_HID / SG_SCORE)
  const uint16_t* vec;          // [K] bf16: x, or h for the down product
  const uint16_t* Ag;           // [N x Kg] gate rows (W_gate or U), or null
  const float* vecg;            // [Kg] fp32 gate vector (low-rank t), or null: the gate uses vec
  int epi;                      // SgEpi
  float* out; void* y; int y_f32; void* hout;
  const float* bias; float bias_scalar; const float* tau; int sel, act;
  const float* colnorm; float* s_buf; float* h_buf; float* g_debug; float* s_debug;
  int seg, rpb, kvec;           // set by sgemv1_plan: item elements, rows per workgroup, staged vector length
};
bool sgemv1_plan(Sgemv1Desc& d, int cus);
hipError_t launch_sgemv1(const Sgemv1Desc& d, hipStream_t s);

// Sparse up / down over the pack at prefill token counts, one eighth of the
// weights per XCD (k_xcd_up: tiles j = r mod 8; k_xcd_down: y column slice r).
struct XcdDesc {
  int M, d, T, E, ntiles, lg_e;   // lg_e = log2 E
  const void* x; const void* w_up; const void* w_down_nm;
  const int32_t* cnt; const uint16_t* idx; const void* val;   // val: bf16 activations a
  float* hp;                      // [M x ntiles x E] h per pack slot
  void* y;
  int route_pass;                 // the extra last workgroup routes the pack
  RouteDesc route;
};
bool xcd_ok(const XcdDesc& u);
// Prefill-shaped MFMA GEMM (128+ tokens): whether it takes a product, the
// launch, and the slice sum of its split-K mode.
bool pf_ok(const GemmDesc& g, const EpiDesc& e);
hipError_t launch_gemm_pf(const GemmDesc& g, const EpiDesc& e, hipStream_t s);
hipError_t launch_pf_ksum(const GemmDesc& g, const EpiDesc& e, hipStream_t s);
constexpr int kPfSplitK = 8;       // K slices of the dense backup's down product
hipError_t launch_xcd_up(const XcdDesc& u, hipStream_t s);     // + the routing pass
hipError_t launch_xcd_down(const XcdDesc& u, hipStream_t s);

// Entries one sparse workgroup holds in LDS (tiles per group * max entries per tile).
constexpr int kUpdownCap = 2048;
__host__ __device__ inline int ud_groups(const UpdownDesc& u) { return (u.F / u.T + u.tiles_per_group - 1) / u.tiles_per_group; }
// Fused sparse up + down over the pack; then the ordered sum of the partial
// rows (skipped by the caller when every token fits one workgroup).
hipError_t launch_updown(const UpdownDesc& u, hipStream_t s);
hipError_t launch_updown_reduce(const UpdownDesc& u, hipStream_t s);

// Decode path (bf16, bias / threshold selection, at most 8 tokens): three
// kernels, all on the whole chip.
//   k_dec_lowrank  t = V x (low-rank gate only), fp32 [M x rank]
//   k_dec_gate     gate rows of one sub-tile (R rows of a TwELL tile) for all
//                  tokens, selection, TwELL pack (look-back across the
//                  sub-tiles of a tile), then u_i = <W_up[i,:], x_t> for the
//                  neurons active for any token: h = a * u into the dense
//                  hidden array, and the sub-tile's union mask
//   k_dec_down     one workgroup per 16-byte column chunk of y: y[:, chunk] =
//                  sum over the hidden list of h * W_down^T[i, chunk], in a
//                  fixed order; the extra last workgroup routes the pack
// Down-projection organisation of the decode path.
//   DEC_CHUNK  gate workgroups compute h of their active neurons into a dense
//              array; k_dec_down: one workgroup per 16-byte column chunk
//   DEC_PART   gate workgroups also sum their down rows into a partial y row;
//              k_dec_reduce adds the partial rows
//   DEC_SPLIT  gate workgroups publish masks and activations only; k_dec_up
//              computes h of the union neurons, 16 at a time, on matrix cores
//              (compact list); k_dec_down2 contracts the list's row slices
//              with h on matrix cores
enum DecMode : int { DEC_CHUNK = 0, DEC_PART = 1, DEC_SPLIT = 2 };
struct DecodeDesc {
  int M, d, F, T, E, K;        // K: gate contraction length (d, or rank)
  int rank;                    // 0: full gate
  int sel;                     // SEL_BIAS / SEL_THRESH
  const void* a_gate;          // W_gate [F x d] or U [F x rank]
  const void* v;               // V [rank x d]
  const void* w_up;            // [F x d]
  const void* w_down_nm;       // [F x d]
  const void* x;               // [M x d]
  void* y;                     // [M x d]
  float* t;                    // [M x rank] low-rank intermediate
  const float* bias; float bias_scalar; const float* tau;
  int32_t* cnt; uint16_t* idx; void* val;   // TwELL pack
  uint64_t* lb;                // per-token look-back words [8 x F / R]
  uint32_t* ctrl;              // control words (look-back epoch, wait limits, error word)
  float* g_debug;              // [M x F] or null
  int R;                       // gate rows per workgroup (divides T)
  int ipw;                     // gate pieces (1 KB of a row) per wave: 1, 2 or 4
  int up;                      // 1: compute the hidden list (forward); 0: pack only
  uint64_t* umask;             // [F / R] neurons of each sub-tile active for any token
  float* hd;                   // [M x F] h of those neurons (column-chunk mode)
  float* part;                 // [F / R x M x d] fp32 partial y rows (partial-row mode)
  int mode;                    // DEC_CHUNK, DEC_PART or DEC_SPLIT (see DecMode)
  float* ad;                   // [M x F] split mode: a = z (active) or 0 for union neurons
  int32_t* ul_total;           // [1] split mode: union-list length
  int32_t* ul_nrn;             // [F] split mode: union neurons, ascending (compact)
  float* ul_h;                 // split mode: hT, bf16 [M][ldh], h per token of each list entry
  int ldh;                     // split mode: row stride of hT (list entries, >= F rounded up to 32)
  int ngroups;                 // split mode: entry groups of the down kernel (partials in part)
  int route_pass;              // k_dec_down: the last workgroup routes the pack
  int nslab;                   // low rank, 2..16 tokens: t as nslab fp32 slabs [nslab][M][rank] (0: t)
  float* tslab;
  RouteDesc route;
};
// Descriptors of several FFNs of one shape for the grouped one-token launches
// (grid.y selects the FFN).
constexpr int kDecGroupMax = 8;
struct DecGroup {
  DecodeDesc d[kDecGroupMax];
};
static_assert(sizeof(DecGroup) <= 4096, "kernel arguments are limited to 4 KiB");
// The split sequence for a group of FFNs of one shape with 2..8 tokens each
// (stage 0: t = V x; 1: the gate; 2: the up products; 3: the down products
// and the ordered sum, whose extra workgroup routes each FFN's pack).
hipError_t launch_dec_split_group(const DecGroup& g, int n, int stage, hipStream_t s);
bool dec_split_group_shape(const DecodeDesc& d);
hipError_t launch_dec_lowrank_group(const DecGroup& g, int n, hipStream_t s);
hipError_t launch_dec_gate_group(const DecGroup& g, int n, hipStream_t s);
hipError_t launch_dec_reduce_group(const DecGroup& g, int n, hipStream_t s);
constexpr int kDecMaxM = 16;       // split sequence; the chunk and partial-row modes stop at 8
// waves of the gate workgroup: 16 for one token; 8 (twice the registers per
// thread) when the up / down accumulators hold several tokens
constexpr int dec_gate_waves(int maxm) { return maxm == 1 ? 16 : 8; }
constexpr int kDecVWaves = 4;      // waves of the low-rank first-stage workgroup
// Whether the gate kernel stages the tokens' x in LDS: a full gate reads it,
// and so do the up products of the partial-row and chunk modes; a low-rank
// gate in split mode or a pack-only pass (up = 0) does not.
__host__ __device__ constexpr bool dec_gate_needs_x(bool lowrank, int mode, int up) {
  return !lowrank || (up != 0 && mode != DEC_SPLIT);
}
// Dynamic LDS bytes of k_dec_gate / k_dec_lowrank for a descriptor.
size_t dec_gate_lds(const DecodeDesc& d);
size_t dec_lowrank_lds(const DecodeDesc& d);
hipError_t launch_dec_lowrank(const DecodeDesc& d, hipStream_t s);
hipError_t launch_dec_gate(const DecodeDesc& d, hipStream_t s);
hipError_t launch_dec_down(const DecodeDesc& d, hipStream_t s);
hipError_t launch_dec_reduce(const DecodeDesc& d, hipStream_t s);
hipError_t launch_dec_up(const DecodeDesc& d, hipStream_t s);
bool dec_split_ok(const DecodeDesc& d);
hipError_t launch_dec_down2(const DecodeDesc& d, hipStream_t s);   // + the group-partial sum
int dec_down2_groups(int d_model, int d_ff);
// Gate rows per decode workgroup for a gate contraction length K, TwELL tile
// width T and m tokens (0 when the decode shape does not apply).
int dec_rows_per_wg(int K, int T, int m, int* ipw, int want_ipw = 0);
int dec_gate_rows(int K, int T, int m, bool lowrank, int* ipw, int want_ipw = 0);

// Mixture-of-experts layer: expert-grouped gather of x (and per-slot bias /
// threshold) and the weighted combination of the experts' outputs.
constexpr int kMoeMaxPairs = 256;   // (token, slot) pairs of one call
struct MoeTable {
  int32_t src[kMoeMaxPairs];        // grouped row r holds pair src[r] = token * topk + slot
  int32_t pos[kMoeMaxPairs];        // pair q = token * topk + slot sits at grouped row pos[q]
  float w[kMoeMaxPairs];            // combine weight of pair q
};
struct MoeDesc {
  int d, m, topk, npairs, dtype;
  const void* x; void* xg;          // [m x d], [npairs x d]
  const float* tau; const float* bias;   // [m x topk] per pair, or null
  float* tg; float* bg;             // [npairs] grouped
  const void* yg; void* y;          // [npairs x d] expert outputs, [m x d]
  MoeTable tab;
};
// Backward pass of the sparse FFN (full ReLU gate, selection held fixed).
// Pair positions: a non-routed token's pack slot (t, tile j, slot s) sits at
// (t * ntiles + j) * E + s; a routed token (dense-list slot r) and neuron i at
// pbase + r * F + i (pbase = m * ntiles * E).
constexpr int kBwBlock = 64;        // tokens per block of the neuron-major index build
struct BwDesc {
  int m, d, F, T, E, ntiles, dtype, sel, nblk, routing;
  const void* x; const void* dy; void* dx;
  const void* w_gate; const void* w_up; const void* w_down_nm;
  const float* bias; float bias_scalar; const float* tau;
  const int32_t* cnt; const uint16_t* idx; const void* val; const uint8_t* route;
  const int32_t* dense_list; const int32_t* n_dense;
  int32_t* slot_of;                 // [m] dense-list slot of a routed token, -1 otherwise
  const float* zr;                  // [m x F] gate g of the routed tokens (slot order), before bias
  int32_t* blk;                     // [nblk x F] pairs per (token block, neuron), then their offsets
  int32_t* colptr;                  // [F + 1] neuron-major start of each neuron's pairs
  int32_t* ent_tok; int32_t* ent_pos;   // neuron-major pairs: token, pair position
  float* du; float* dz;             // per pair position
  float* dxp;                       // [splits x m x d] fp32 partial dx rows (few tokens), or null
  uint16_t* duz;                    // [m x 2F] bf16 rows (du | dz) for the matrix-core dx, or null
  long long pbase;
  float* dw_gate; float* dw_up; float* dw_down;   // [F x d] fp32, accumulated
};
hipError_t launch_bw_slots(const BwDesc& d, hipStream_t s);
hipError_t launch_bw_count(const BwDesc& d, hipStream_t s);
hipError_t launch_bw_scan(const BwDesc& d, hipStream_t s);
hipError_t launch_bw_fill(const BwDesc& d, hipStream_t s);
hipError_t launch_bw_neuron(const BwDesc& d, hipStream_t s);
hipError_t launch_bw_dx(const BwDesc& d, hipStream_t s);
hipError_t launch_bw_duz(const BwDesc& d, hipStream_t s);
// From this many tokens (bf16) dx is a matrix-core GEMM of the dense (du | dz)
// rows with [W_up; W_gate] instead of per-token row gathers.
constexpr int kBwDxDenseMin = 512;
// Splits of each token's neuron list in the dx kernel (more workgroups for
// few tokens; at most kBwDxPartRows partial rows).
constexpr int kBwDxMaxSplit = 16;
constexpr int kBwDxPartRows = 512;
int bw_dx_splits(int m);
hipError_t launch_moe_gather(const MoeDesc& d, hipStream_t s);
hipError_t launch_moe_combine(const MoeDesc& d, hipStream_t s);
// Slices of d of the matrix-core first stage for m tokens (0: the VALU kernel).
int dec_lowrank_slabs(int m, int d_model, int rank, int want);

}  // namespace ffn
