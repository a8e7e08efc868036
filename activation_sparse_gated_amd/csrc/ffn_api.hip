// C ABI of the sparse gated FFN library: argument checks, workspace layout,
// kernel planning and launches. Everything here runs on the host; every step
// of the computation runs in the kernels of k_gate / k_updown / k_topk.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/ffn_sparse.h"
#include "kernels.cuh"
#include "gemm_core.cuh"

using namespace ffn;

namespace ffn {
thread_local LaunchEvents tl_launch_events = {nullptr, nullptr};
}  // namespace ffn

// ---------------------------------------------------------------- scratch
// Per-call device memory of ffn_sparse_forward_noalloc, for callers that
// cannot allocate: a fixed-size array that each GPU the library runs on holds
// until the process ends, shared by every no-allocation call on that GPU.
// Host code never uses the array's name as an address: each device's copy is
// resolved with hipGetSymbolAddress once, with that device current.
//   [0, 256)                  control words (pass epoch, wait limits, error word)
//   [256, +kScrLbBytes)       look-back words of the decode gate, kDecMaxM tokens x
//                             kScrMaxF / 2 sub-tiles (epoch-tagged, cleared once)
//   then kScrMaxF list ids, the list length, and the per-call regions (low-rank
//   slabs and t, sub-tile masks, hidden values, partial y rows, list h)
constexpr size_t kScratchBytes = 20u << 20;
constexpr int kScrMaxF = 32768;
constexpr size_t kScrCtrlBytes = 256;
constexpr size_t kScrLbBytes = (size_t)kDecMaxM * (kScrMaxF / 2) * sizeof(uint64_t);
constexpr size_t kScrIdsBytes = (size_t)kScrMaxF * sizeof(int32_t);
constexpr size_t kScrFixedBytes = kScrCtrlBytes + kScrLbBytes + kScrIdsBytes + 256;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of `scratch`; on the first request for a device its
// address is resolved and its fixed regions are cleared on `s` (which is then
// synchronised), the wait limit set.
hipError_t scratch_for_device(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    uint32_t* w = reinterpret_cast<uint32_t*>(ptr);
    e = launch_fill_u32(w, 0u, kScrFixedBytes / 4, s);
    if (e == hipSuccess) e = launch_fill_u32(w + CTRL_SPIN_LIMIT, kDefaultSpinLimit, 1, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Error word of this device's scratch (0 when it has none yet).
uint32_t scratch_error_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  void* ptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev];
  }
  uint32_t err = 0;
  if (ptr && hipMemcpy(&err, reinterpret_cast<uint32_t*>(ptr) + CTRL_ERR, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess)
    return 1;
  return err;
}
}  // namespace

namespace {

constexpr size_t kAlign = 256;
constexpr int kCtrlWords = 64;
constexpr int kTicketWords = 1 << 16;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int esize_of(int dtype) { return dtype == FFN_F32 ? 4 : 2; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Rows per tile of the gate GEMM: the largest of 128/64/32/16 that divides the
// TwELL tile and still leaves at least `want` workgroups.
int pick_nt(int nrows, int nmat, int T, int mblocks, int want, bool f32) {
  const int cands[4] = {128, 64, 32, 16};
  int best = 0;
  for (int nt : cands) {
    if (f32 && nt > 64) continue;
    if (nmat == 2 && nt < 32) continue;
    const int rpm = nt / nmat;
    if (T > 0 && T % rpm != 0) continue;
    if (nrows % rpm != 0) continue;
    best = nt;  // keeps the smallest valid so far (loop goes large -> small)
    if ((nrows / rpm) * mblocks >= want) return nt;
  }
  return best;
}

int pick_mt(int m) { return m <= 16 ? 16 : (m <= 32 ? 32 : 64); }

// Token counts up to this are "decode": the sparse kernel also evaluates
// routed tokens (no extra launches); larger counts use the dense backup GEMMs.
constexpr int kDecodeMaxM = 64;

// Token counts of the masked dense sequence: above the decode kernels' 16
// tokens the union of the tokens' active neurons covers most rows (at 10%
// density, 1 - 0.9^17 = 83%; 97% at 32 tokens), so a sparse pass cannot read
// fewer weight bytes than the dense products, and below the prefill shapes
// (128 tokens) the products are weight streams.
constexpr int kMaskedDenseMaxM = 127;
// Up to 256 tokens the masked dense sequence also replaces the general path
// of configurations whose pack the XCD-sliced pair cannot hold (more than 64
// TwELL tiles, or 1024 slots a token), where the per-token sparse kernel would
// gather every union row once per token (LoPA, 256 tokens: 695 us against
// 293 us for the dense FFN).
constexpr int kMaskedDenseMaxMNoXcd = 256;

// Whether the XCD-sliced pair takes this configuration's pack (its shape
// limits only; the token count and pointers are checked at the call).
bool xcd_config_ok(const ffn_sparse_config& c) {
  if (c.dtype != FFN_BF16 || c.sel == FFN_SEL_TOPK_WINA || c.tile_w <= 0 || c.ell_w <= 0) return false;
  static char dummy[16];
  XcdDesc x{};
  x.M = 128;
  x.d = c.d_model;
  x.T = c.tile_w;
  x.E = c.ell_w;
  x.ntiles = c.d_ff / c.tile_w;
  x.lg_e = 0;
  while ((1 << x.lg_e) < x.E) ++x.lg_e;
  x.x = x.w_up = x.w_down_nm = dummy;
  x.cnt = reinterpret_cast<const int32_t*>(dummy);
  x.idx = reinterpret_cast<const uint16_t*>(dummy);
  x.val = dummy;
  x.hp = reinterpret_cast<float*>(dummy);
  x.y = dummy;
  return xcd_ok(x);
}

// Largest token count of the masked dense sequence for a configuration.
int masked_dense_max_m(const ffn_sparse_config& c) {
  return xcd_config_ok(c) ? kMaskedDenseMaxM : kMaskedDenseMaxMNoXcd;
}

struct Workspace {
  uint32_t* ctrl;       // kCtrlWords control words + kTicketWords tickets
  void* wdown_alt;      // the W_down layout the caller did not pass
  float* colnorm;       // [F]
  float* lr_slabs;       // [kMaxSlabs x max_m x rank] first-stage partial slabs
  float* lr_t;           // [max_m x rank] summed intermediate
  float* g_ext;          // [max_m x F] low-rank gate values of the dense paths
  float* wina_s;         // [max_m x F]
  float* wina_h;         // [max_m x F]
  uint64_t* lb;          // [max_m x F / 16]
  float* ud_partial;     // [ud_rows x d]
  size_t ud_rows;
  void* hbuf;            // [max_m x F] dense hidden
  uint64_t* dec_lb;      // [kDecMaxM x F / 2] per-token look-back words of the decode gate
  uint64_t* umask;       // [F / 2] decode sub-tiles: neurons active for any token
  float* hd;             // [kDecMaxM x F] decode hidden values (column-chunk mode)
  float* dec_part;       // [F / R x min(max_m, 8) x d] decode partial y rows
  size_t dec_part_rows;  // rows of d floats in dec_part
  float* xh;             // [M x F / T x E] prefill: h per pack slot (XCD-sliced up / down)
  float* kpart;          // [kPfSplitK x M x d] prefill dense backup: split-K partials (or null)
  int32_t* ul_total;     // [1] decode split mode: union-list length
  int32_t* ul_nrn;       // [F] decode split mode: union neurons
  float* ul_h;           // decode split mode: hT, bf16 [kDecMaxM][F rounded up to 32]
  uint16_t* in_wt;       // input-side gate: W^T [d x N] (N = F, or rank)
  float* in_norm;        // input-side gate: [d] column norms of W_gate (or V)
  int32_t* in_kidx;      // input-side gate: [max_m x in_keep] kept channels
  uint16_t* in_kval;     // input-side gate: [max_m x in_keep] their x values
  float* in_part;        // input-side gate: [groups x max_m x N] partial sums
  int in_groups;
  size_t total;
};

constexpr int kMaxSlabs = 8;
// Partial y rows of the sparse kernel: enough for 4 per CU, and for every
// token at the coarsest grouping (64 tiles per workgroup).
size_t ud_rows_for(const ffn_sparse_config& c, int cus) {
  const size_t ntiles = c.d_ff / c.tile_w;
  const size_t per_tile = std::max(1, std::max(c.ell_w, c.tile_w));
  const size_t gmin = std::max<size_t>(1, std::min<size_t>(std::min<size_t>(ntiles, 64), kUpdownCap / per_tile));
  return std::max<size_t>((size_t)4 * cus, (size_t)c.max_m * ((ntiles + gmin - 1) / gmin));
}

// Carves the workspace (base may be null to only compute the size).
Workspace carve(const ffn_sparse_config& c, char* base, int cus) {
  Workspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  const size_t es = esize_of(c.dtype);
  const size_t F = c.d_ff, d = c.d_model, r = c.rank, M = c.max_m;
  w.ctrl = (uint32_t*)take((kCtrlWords + kTicketWords) * sizeof(uint32_t));
  w.wdown_alt = take(F * d * es);
  w.colnorm = (float*)take(F * sizeof(float));
  w.lr_slabs = (float*)take(std::max<size_t>(1, kMaxSlabs * M * r) * sizeof(float));
  w.lr_t = (float*)take(std::max<size_t>(1, M * r) * sizeof(float));
  // gate values [tokens x F] fp32: the dense paths of a low-rank gate, and
  // the masked dense sequence (17..127 tokens; see masked_dense_ok)
  const bool md = c.dtype == FFN_BF16 && c.sel != FFN_SEL_TOPK_WINA && c.in_keep == 0 && M > (size_t)kDecMaxM;
  const size_t md_rows = std::min<size_t>(M, masked_dense_max_m(c));
  w.g_ext = (float*)take(r ? M * F * sizeof(float) : (md ? md_rows * F * sizeof(float) : 16));
  const bool topk = c.sel == FFN_SEL_TOPK_WINA;
  w.wina_s = (float*)take(topk ? M * F * sizeof(float) : 16);
  w.wina_h = (float*)take(topk ? M * F * sizeof(float) : 16);
  w.lb = (uint64_t*)take(M * (F / 16) * sizeof(uint64_t));
  w.ud_rows = ud_rows_for(c, cus);
  w.ud_partial = (float*)take(w.ud_rows * d * sizeof(float));
  w.hbuf = take(M * F * es);
  w.dec_lb = (uint64_t*)take((size_t)kDecMaxM * (F / 2) * sizeof(uint64_t));
  w.umask = (uint64_t*)take((F / 2) * sizeof(uint64_t));
  w.hd = (float*)take(F * kDecMaxM * sizeof(float));
  {
    // the smallest sub-tile (most partial rows) over the token counts 1..8
    int R = 0;
    if (c.dtype == FFN_BF16 && c.sel != FFN_SEL_TOPK_WINA) {
      const int K = c.rank ? c.rank : c.d_model;
      const int r1 = dec_rows_per_wg(K, c.tile_w, 1, nullptr), r2 = dec_rows_per_wg(K, c.tile_w, 2, nullptr);
      R = (r1 && r2) ? std::min(r1, r2) : (r1 ? r1 : r2);
    }
    // partial rows of the gate sub-tiles (partial-row mode, up to 8 tokens)
    // or of the down kernel's entry groups (split mode, up to 16 tokens; also
    // top-k selection's list-driven down product for one token)
    const size_t rows_part = R ? (F / R) * std::min<size_t>(M, 8) : 0;
    const size_t rows_split = c.dtype == FFN_BF16 ? 32 * std::min<size_t>(M, kDecMaxM) : 0;
    const size_t rows = std::max(rows_part, rows_split);
    w.dec_part = (float*)take(rows ? rows * d * sizeof(float) : 16);
    w.dec_part_rows = rows;
  }
  // split-K partials of the dense backup's down product at prefill sizes
  const bool can_route = !topk && c.ell_w < c.tile_w;
  w.kpart = (float*)(M >= 128 && can_route && c.dtype == FFN_BF16 ? take((size_t)kPfSplitK * M * d * sizeof(float))
                                                                    : nullptr);
  // h per pack slot of the XCD-sliced prefill up / down pair
  w.xh = (float*)take(M >= 128 && !topk ? M * (F / c.tile_w) * std::max(1, c.ell_w) * sizeof(float) : 16);
  w.ul_total = (int32_t*)take(sizeof(int32_t));
  w.ul_nrn = (int32_t*)take(F * sizeof(int32_t));
  w.ul_h = (float*)take((size_t)kDecMaxM * ((F + 31) / 32 * 32) * sizeof(uint16_t));
  if (c.in_keep > 0) {
    const size_t N = r ? r : F, k = c.in_keep;
    w.in_groups = in_groups((int)N, (int)k);
    w.in_wt = (uint16_t*)take(d * N * sizeof(uint16_t));
    w.in_norm = (float*)take(d * sizeof(float));
    w.in_kidx = (int32_t*)take(M * k * sizeof(int32_t));
    w.in_kval = (uint16_t*)take(M * k * sizeof(uint16_t));
    w.in_part = (float*)take((size_t)w.in_groups * M * N * sizeof(float));
  }
  w.total = off;
  return w;
}

int device_lds_max() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
    return v;
  return 64 * 1024;
}

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  return cus;
}

}  // namespace

// Path switches (0 = automatic), read once at init from the environment; each
// forces a kernel sequence the parity tests also run:
// FFN_SPARSE_NO_DECODE (1: the general kernels at 1..16 tokens too),
// FFN_SPARSE_DEC_MODE (1 + DecMode: force the decode down-projection
// organisation), FFN_SPARSE_NO_PREFILL_GEMM (1: the decode-shaped MFMA kernel
// for 128+ tokens as well), FFN_SPARSE_NO_TOPK_DOWN (1: top-k selection's down
// product through the per-token TwELL kernel), FFN_SPARSE_NO_XCD (1: the
// per-token sparse kernel at prefill token counts too),
// FFN_SPARSE_NO_MASKED_DENSE (1: the general sequence at 17..127 tokens).
// Launch-shape overrides for tuning exist only in a library compiled with
// -DFFN_SPARSE_TUNING (FFN_SPARSE_GATE_NT, _GATE_WAVES, _UD_SPLIT, _UD_GROUP,
// _UD_WAVES, _V_KS, _NO_GEMV, _LR_SLABS, _DEC_IPW, _UD_ORDER); the product
// build ignores them, so a caller's environment cannot select a launch shape
// the tests do not run. None changes the result beyond floating-point
// summation order.
struct Tuning {
  int gate_nt = 0, gate_waves = 0, ud_split = 0, ud_group = 0, ud_waves = 0, v_ks = 0, no_gemv = 0, no_decode = 0, dec_mode = 0, no_pf = 0,
      no_topk_down = 0, no_xcd = 0, lr_slabs = 0, dec_ipw = 0, ud_order = 0, no_masked_dense = 0;
};

static int env_int(const char* name) {
  const char* v = getenv(name);
  return v ? atoi(v) : 0;
}

struct ffn_sparse_handle {
  ffn_sparse_config cfg;
  const void *w_gate, *u, *v, *w_up, *w_down_om, *w_down_nm;
  Workspace ws;
  int cus;
  int lds_max;
  Tuning tune;
  // set when a launch failed part-way through a call or a bounded wait gave
  // up: the look-back words may then be out of step with the epoch, so every
  // later call returns FFN_E_HIP until the handle is re-initialised
  bool failed = false;
  // timing
  bool timing = false;
  int cap = 0;
  std::vector<hipEvent_t> ev[FFN_K_COUNT][2];
  int used[FFN_K_COUNT] = {};
};

namespace {

// Per-kernel timing: the next kernel launched in the scope records the pair
// of events from its own dispatch (see ffn_launch); a scope that launched
// nothing records nothing.
struct Timed {
  ffn_sparse_handle* h;
  int kind;
  bool on;
  Timed(ffn_sparse_handle* hh, int k, hipStream_t) : h(hh), kind(k) {
    on = h->timing && h->used[kind] < h->cap;
    if (on) tl_launch_events = LaunchEvents{h->ev[kind][0][h->used[kind]], h->ev[kind][1][h->used[kind]]};
  }
  ~Timed() {
    if (!on) return;
    if (tl_launch_events.start == nullptr) h->used[kind]++;   // a launch took the events
    else tl_launch_events = LaunchEvents{nullptr, nullptr};
  }
};

ffn_status hip_status(hipError_t e) { return e == hipSuccess ? FFN_OK : FFN_E_HIP; }

GemmDesc gemm_base(const ffn_sparse_handle* h) {
  GemmDesc g{};
  g.dtype = h->cfg.dtype;
  g.nmat = 1;
  g.ks = 1;
  g.b_nsum = 1;
  g.nwaves = 4;
  g.ctrl = h->ws.ctrl;
  g.bmode = B_NATIVE;
  g.no_pf = h->tune.no_pf;
  return g;
}

// Decode GEMV shape (bf16, M <= 8, K <= 4096): rows per workgroup from
// 128..4 (dividing the TwELL tile T when T > 0), the largest that still gives
// `want` workgroups; 16 waves for tiles of 64+ rows, else 4.
bool plan_gemv(GemmDesc& g, const ffn_sparse_handle* h, int T, int want) {
  if (g.dtype != FFN_BF16 || g.M > 8 || g.M < 1) return false;
  const int cands[6] = {128, 64, 32, 16, 8, 4};
  int best = 0;
  for (int nt : cands) {
    if (nt < 2 * g.nmat) continue;
    const int rpm = nt / g.nmat;
    if (T > 0 && (T % nt != 0)) continue;
    if (g.nrows % rpm != 0) continue;
    best = nt;
    if ((g.nrows / rpm) >= want) break;
  }
  if (h->tune.gate_nt && T > 0 && T % h->tune.gate_nt == 0 && h->tune.gate_nt <= 128) best = h->tune.gate_nt;
  if (best == 0) return false;
  GemmDesc t = g;
  t.gemv = 1;
  t.nt = best;
  t.mt = 16;
  t.ks = 1;
  t.nwaves = best >= 64 ? 16 : 4;
  if (T > 0 && (h->tune.gate_waves == 4 || h->tune.gate_waves == 16)) t.nwaves = h->tune.gate_waves;
  if (!gemv_ok(t)) return false;
  g = t;
  return true;
}

// Tile shape of a GEMM without a TwELL constraint: rows per workgroup from
// 128/64/32/16 (the largest that still gives >= cus workgroups), 16 waves
// when there are few workgroups (more bytes in flight per CU), else 4.
bool plan_plain(GemmDesc& g, const ffn_sparse_handle* h) {
  if (!h->tune.no_gemv && plan_gemv(g, h, 0, 3 * h->cus / 4)) return true;
  g.gemv = 0;
  const bool f32 = g.dtype == FFN_F32;
  g.mt = f32 ? 16 : pick_mt(g.M);
  const int mblocks = ceil_div(g.M, g.mt);
  g.nt = pick_nt(g.nrows, g.nmat, 0, mblocks, h->cus, f32);
  if (g.nt == 0) return false;
  const int wgs = g.nrows * g.nmat / g.nt * mblocks;
  g.nwaves = (!f32 && wgs <= 2 * h->cus) ? 16 : 4;
  g.ks = 1;
  return true;
}

// The gate with the TwELL epilogue: one workgroup per TwELL tile when there
// are enough tiles (no look-back), else sub-tiles of the TwELL tile.
bool plan_twell(GemmDesc& g, const ffn_sparse_handle* h) {
  const auto& c = h->cfg;
  if (!h->tune.no_gemv && plan_gemv(g, h, c.tile_w, 3 * h->cus / 4)) return true;
  g.gemv = 0;
  const bool f32 = g.dtype == FFN_F32;
  g.mt = f32 ? 16 : pick_mt(g.M);
  const int mblocks = ceil_div(g.M, g.mt);
  const int T = c.tile_w;
  if (!f32 && T <= 128 && (c.d_ff / T) * mblocks >= 3 * h->cus / 4) {
    g.nt = T;
  } else {
    // sub-tiles until about three quarters of the CUs have a workgroup (LoPA,
    // 64 tokens: 64-row sub-tiles, 224 workgroups: gate 48.9 -> 35.4 us
    // against whole 128-row tiles)
    g.nt = pick_nt(c.d_ff, 1, T, mblocks, 3 * h->cus / 4, f32);
  }
  if (h->tune.gate_nt && T % h->tune.gate_nt == 0 && h->tune.gate_nt <= (f32 ? 64 : 128)) g.nt = h->tune.gate_nt;
  if (g.nt == 0) return false;
  const int wgs = c.d_ff / g.nt * mblocks;
  g.nwaves = (!f32 && wgs <= 2 * h->cus) ? 16 : 4;
  if (!f32 && (h->tune.gate_waves == 4 || h->tune.gate_waves == 16)) g.nwaves = h->tune.gate_waves;
  g.ks = 1;
  return true;
}

bool pack_ok(const ffn_twell_pack* p) {
  return p && p->cnt && p->idx && p->val && p->route && p->dense_list && p->n_dense &&
         aligned16(p->cnt) && aligned16(p->idx) && aligned16(p->val);
}

ffn_status check_call(const ffn_sparse_handle* h, const void* x, int m, const float* tau, int k) {
  if (!h) return FFN_E_INVALID;
  if (m < 0 || m > h->cfg.max_m) return FFN_E_INVALID;
  if (m > 0 && (!x || !aligned16(x))) return FFN_E_INVALID;
  if (h->cfg.sel == FFN_SEL_THRESH && m > 0 && !tau) return FFN_E_INVALID;
  if (h->cfg.sel == FFN_SEL_TOPK_WINA && (k < 0 || k > h->cfg.d_ff)) return FFN_E_INVALID;
  return FFN_OK;
}

EpiDesc epi_base(const ffn_sparse_handle* h, const float* bias, float bias_scalar, const float* tau) {
  EpiDesc e{};
  e.F = h->cfg.d_ff;
  e.out_f32 = h->cfg.dtype == FFN_F32;
  e.bias = bias;
  e.bias_scalar = bias_scalar;
  e.tau = tau;
  e.sel = h->cfg.sel;
  e.act = h->cfg.act;
  e.T = h->cfg.tile_w;
  e.E = h->cfg.ell_w;
  return e;
}

// One-token dense stream (k_sgemv.hip) for bf16 configs, m = 1 without a
// gathered token list; false when it does not apply.
bool one_token_stream(const ffn_sparse_handle* h, int m, const int32_t* gather, const int32_t* m_dev) {
  return m == 1 && !gather && !m_dev && h->cfg.dtype == FFN_BF16 && !h->tune.no_gemv;
}

Sgemv1Desc sg_base(const ffn_sparse_handle* h, const float* bias, float bias_scalar, const float* tau) {
  Sgemv1Desc d{};
  d.bias = bias;
  d.bias_scalar = bias_scalar;
  d.tau = tau;
  d.sel = h->cfg.sel;
  d.act = h->cfg.act;
  return d;
}

// First stage of the low-rank gate, t = V x, for `m` token slots (optionally
// gathered): ks workgroups split K and each writes an fp32 slab
// [m x rank] at lr_slabs + slab * max_m * rank. Returns the slab count.
int run_lowrank_v(ffn_sparse_handle* h, const void* x, int m, const int32_t* gather, const int32_t* m_dev,
                  hipStream_t s, hipError_t* err) {
  const auto& c = h->cfg;
  GemmDesc g = gemm_base(h);
  g.A0 = h->v;
  g.nrows = c.rank;
  g.lda = c.d_model;
  g.K = c.d_model;
  g.B = x;
  g.ldb = c.d_model;
  g.M = m;
  g.gather = gather;
  g.m_dev = m_dev;
  if (one_token_stream(h, m, gather, m_dev)) {      // one token: a plain weight stream
    Sgemv1Desc d = sg_base(h, nullptr, 0.f, nullptr);
    d.N = c.rank;
    d.K = c.d_model;
    d.A = reinterpret_cast<const uint16_t*>(h->v);
    d.vec = reinterpret_cast<const uint16_t*>(x);
    d.epi = SG_OUT;
    d.out = h->ws.lr_slabs;
    if (sgemv1_plan(d, h->cus)) {
      Timed tm(h, FFN_K_LOWRANK_V, s);
      *err = launch_sgemv1(d, s);
      return 1;
    }
  }
  if (!plan_plain(g, h)) {
    *err = hipErrorInvalidValue;
    return 0;
  }
  if (g.gemv) {                                   // decode: no K split needed
    EpiDesc e{};
    e.kind = EPI_STORE_F32;
    e.F = c.rank;
    e.out = h->ws.lr_slabs;
    e.ldo = c.rank;
    e.out_slab = (long long)c.max_m * c.rank;
    Timed tm(h, FFN_K_LOWRANK_V, s);
    *err = launch_gemm(g, e, s);
    return 1;
  }
  // rank rows are few, so ks workgroups split K (4 waves each, at least two
  // 32-element chunks per wave) until about one workgroup per CU streams V;
  // each writes an fp32 slab, and the slabs are summed once, in order
  // (LoPA, 64 tokens: 8 slabs, 8.8 -> 5.1 us against 2)
  int ks = 1;
  if (c.dtype == FFN_BF16) {
    g.nwaves = 4;
    const int wgs = g.nrows / g.nt * ceil_div(m, g.mt);
    const int kch = g.K / 32;
    while (wgs * ks < h->cus && ks < 8 && kch / (ks * 2 * g.nwaves) >= 2) ks *= 2;
    if (h->tune.v_ks > 0) {
      int want = h->tune.v_ks;
      ks = (want >= 8) ? 8 : (want >= 4 ? 4 : (want >= 2 ? 2 : 1));
      while (ks > 1 && kch / (ks * g.nwaves) < 1) ks /= 2;
    }
  }
  g.ks = ks;
  EpiDesc e{};
  e.kind = EPI_STORE_F32;
  e.F = c.rank;
  e.out = h->ws.lr_slabs;
  e.ldo = c.rank;
  e.out_slab = (long long)c.max_m * c.rank;
  Timed tm(h, FFN_K_LOWRANK_V, s);
  *err = launch_gemm(g, e, s);
  return ks;
}

// Sums the first stage's slabs into slab 0 once (in slab order), so that the
// gate GEMM reads t as one slab; returns the slab count left (1).
int collapse_slabs(ffn_sparse_handle* h, int m, int nslabs, hipStream_t s, hipError_t* err) {
  if (nslabs <= 1) return nslabs;
  Timed tm(h, FFN_K_LOWRANK_V, s);
  *err = launch_slab_sum(h->ws.lr_slabs, nslabs, (size_t)h->cfg.max_m * h->cfg.rank, (size_t)m * h->cfg.rank, s);
  return 1;
}

// Points a GEMM's B operand at the first-stage slabs (summed on load).
void b_from_slabs(GemmDesc& g, const ffn_sparse_handle* h, int nslabs) {
  g.B = h->ws.lr_slabs;
  g.ldb = h->cfg.rank;
  g.K = h->cfg.rank;
  g.bmode = h->cfg.dtype == FFN_BF16 ? B_F32_SPLIT : B_NATIVE;
  g.b_nsum = nslabs;
  g.b_slab = (long long)h->cfg.max_m * h->cfg.rank;
}

// Dense hidden h (bf16/fp32 [slots x F] in hbuf) for `m` slots; gathered when
// `list` is set (dense backup) with the device count m_dev.
hipError_t run_dense_hidden(ffn_sparse_handle* h, const void* x, int m, const int32_t* list,
                            const int32_t* m_dev, const float* bias, float bias_scalar,
                            const float* tau, int kind, hipStream_t s, bool keep_g = false, int gate_kind = -1) {
  const auto& c = h->cfg;
  if (one_token_stream(h, m, list, m_dev)) {
    // one token: the up rows with the gate rows (W_gate with x, or U with
    // t = V x) in one stream, h written as bf16
    Sgemv1Desc d = sg_base(h, bias, bias_scalar, tau);
    d.N = c.d_ff;
    d.K = c.d_model;
    d.A = reinterpret_cast<const uint16_t*>(h->w_up);
    d.vec = reinterpret_cast<const uint16_t*>(x);
    d.epi = SG_HID;
    d.hout = h->ws.hbuf;
    if (c.rank == 0) {
      d.Ag = reinterpret_cast<const uint16_t*>(h->w_gate);
      d.Kg = c.d_model;
    } else {
      d.Ag = reinterpret_cast<const uint16_t*>(h->u);
      d.Kg = c.rank;
      d.vecg = h->ws.lr_slabs;
    }
    if (sgemv1_plan(d, h->cus)) {
      if (c.rank) {
        hipError_t err = hipSuccess;
        const int nslabs = run_lowrank_v(h, x, m, nullptr, nullptr, s, &err);
        if (err != hipSuccess) return err;
        if (nslabs != 1) return hipErrorInvalidValue;   // the one-token first stage writes t as one slab
      }
      Timed tm(h, kind, s);
      return launch_sgemv1(d, s);
    }
  }
  EpiDesc e = epi_base(h, bias, bias_scalar, tau);
  e.kind = EPI_DENSE_H;
  e.tok_of = list;
  e.hout = h->ws.hbuf;
  e.ldh = c.d_ff;
  GemmDesc g = gemm_base(h);
  g.M = m;
  g.gather = list;
  g.m_dev = m_dev;
  if (c.rank == 0) {
    g.A0 = h->w_gate;
    g.A1 = h->w_up;
    g.nmat = 2;
    g.nrows = c.d_ff;
    g.lda = c.d_model;
    g.K = c.d_model;
    g.B = x;
    g.ldb = c.d_model;
    if (keep_g) e.g_debug = h->ws.g_ext;           // the gate values [m x F], for a pack built from them
    if (!plan_plain(g, h)) return hipErrorInvalidValue;
    Timed tm(h, kind, s);
    return launch_gemm(g, e, s);
  }
  // low-rank gate: t = V x (slabs), g = U t (fp32 into g_ext), then the up GEMM
  hipError_t err = hipSuccess;
  int nslabs = run_lowrank_v(h, x, m, list, m_dev, s, &err);
  if (err != hipSuccess) return err;
  nslabs = collapse_slabs(h, m, nslabs, s, &err);
  if (err != hipSuccess) return err;
  {
    GemmDesc gu = gemm_base(h);
    gu.A0 = h->u;
    gu.nrows = c.d_ff;
    gu.lda = c.rank;
    gu.M = m;
    gu.m_dev = m_dev;
    b_from_slabs(gu, h, nslabs);
    if (!plan_plain(gu, h)) return hipErrorInvalidValue;
    EpiDesc eg{};
    eg.kind = EPI_STORE_F32;
    eg.F = c.d_ff;
    eg.out = h->ws.g_ext;
    eg.ldo = c.d_ff;
    Timed tm(h, gate_kind >= 0 ? gate_kind : kind, s);
    err = launch_gemm(gu, eg, s);
    if (err != hipSuccess) return err;
  }
  g.A0 = h->w_up;
  g.nrows = c.d_ff;
  g.lda = c.d_model;
  g.K = c.d_model;
  g.B = x;
  g.ldb = c.d_model;
  e.g_ext = h->ws.g_ext;
  if (!plan_plain(g, h)) return hipErrorInvalidValue;
  Timed tm(h, kind, s);
  return launch_gemm(g, e, s);
}

// y rows = W_down h for `m` slots of hbuf (scattered through `list`).
// y = A x for m tokens through the library's dense GEMM kernels (bf16, K a
// multiple of 32), for entry points that hold no FFN handle (the GSI linear
// map's dense baseline): a handle with the default launch shapes plans it.
hipError_t dense_rows_impl(const void* A, int nrows, int K, const void* x, int m, void* y, int ldy, int cus,
                           hipStream_t s) {
  ffn_sparse_handle h{};
  h.cfg.dtype = FFN_BF16;
  h.cus = cus;
  GemmDesc g = gemm_base(&h);
  g.A0 = A;
  g.nrows = nrows;
  g.lda = K;
  g.K = K;
  g.B = x;
  g.ldb = K;
  g.M = m;
  if (K % 32 != 0 || !plan_plain(g, &h) || g.ks != 1) return hipErrorInvalidValue;
  EpiDesc e{};
  e.kind = EPI_Y;
  e.F = nrows;
  e.out_f32 = 0;
  e.y = y;
  e.ldy = ldy;
  return launch_gemm(g, e, s);
}

hipError_t run_dense_down(ffn_sparse_handle* h, int m, const int32_t* list, const int32_t* m_dev,
                          void* y, int kind, hipStream_t s) {
  const auto& c = h->cfg;
  if (one_token_stream(h, m, list, m_dev)) {         // one token: the output-major rows against h
    Sgemv1Desc d = sg_base(h, nullptr, 0.f, nullptr);
    d.N = c.d_model;
    d.K = c.d_ff;
    d.A = reinterpret_cast<const uint16_t*>(h->w_down_om);
    d.vec = reinterpret_cast<const uint16_t*>(h->ws.hbuf);
    d.epi = SG_Y;
    d.y = y;
    if (sgemv1_plan(d, h->cus)) {
      Timed tm(h, kind, s);
      return launch_sgemv1(d, s);
    }
  }
  GemmDesc g = gemm_base(h);
  g.A0 = h->w_down_om;
  g.nrows = c.d_model;
  g.lda = c.d_ff;
  g.K = c.d_ff;
  g.B = h->ws.hbuf;
  g.ldb = c.d_ff;
  g.M = m;
  g.m_dev = m_dev;
  if (!plan_plain(g, h)) return hipErrorInvalidValue;
  // K-split partial slabs of the skinny kernel: the sparse kernel's partial-row
  // buffer, which no kernel of a dense down product's call uses
  g.skpart = h->ws.ud_partial;
  g.skpart_rows = (int)std::min<size_t>(h->ws.ud_rows, 1 << 20);
  EpiDesc e{};
  e.kind = EPI_Y;
  e.F = c.d_model;
  e.out_f32 = c.dtype == FFN_F32;
  e.y = y;
  e.ldy = c.d_model;
  e.yrows = list;
  // dense backup at prefill sizes: few routed tokens (a device-side count)
  // leave most 128 x 128 tiles empty, so K is split kPfSplitK ways and the
  // slices are summed in order by a second kernel
  if (list && m_dev && h->ws.kpart && !h->tune.no_pf) {
    GemmDesc gp = g;
    gp.ks = kPfSplitK;
    gp.kpart = h->ws.kpart;
    gp.kpart_m = c.max_m;
    if (pf_ok(gp, e)) {
      {
        Timed tm(h, kind, s);
        hipError_t err = launch_gemm_pf(gp, e, s);
        if (err != hipSuccess) return err;
      }
      Timed tm(h, kind, s);
      return launch_pf_ksum(gp, e, s);
    }
  }
  Timed tm(h, kind, s);
  return launch_gemm(g, e, s);
}

RouteDesc route_desc(const ffn_sparse_handle* h, int m, const ffn_twell_pack* p) {
  RouteDesc r{};
  r.M = m;
  r.ntiles = h->cfg.d_ff / h->cfg.tile_w;
  r.E = h->cfg.ell_w;
  r.cnt = p->cnt;
  r.route = p->route;
  r.dense_list = p->dense_list;
  r.n_dense = p->n_dense;
  r.ctrl = h->ws.ctrl;
  return r;
}

// Gate pass writing cnt / idx / val (no routing; see run_route / updown).
// topk_out (top-k selection only): 0 the pack alone; 1 also the kept neurons
// as the one-token list of the list-driven down kernel; 2 also the masked h
// rows in hbuf for a dense down product.
ffn_status gate_pack_core(ffn_sparse_handle* h, const void* x, int m, const float* bias, float bias_scalar,
                          const float* tau, int k, ffn_twell_pack* pack, float* g_debug, float* s_debug,
                          hipStream_t s, bool* routed_by_topk, int topk_out = 0) {
  const auto& c = h->cfg;
  *routed_by_topk = false;
  EpiDesc e = epi_base(h, bias, bias_scalar, tau);
  e.g_debug = g_debug;
  e.s_debug = s_debug;
  e.cnt = pack->cnt;
  e.idx = pack->idx;
  e.val = pack->val;
  e.lb = h->ws.lb;
  e.lb_ld = h->cfg.max_m;
  GemmDesc g = gemm_base(h);
  g.M = m;
  if (c.sel == FFN_SEL_TOPK_WINA) {
    g.A0 = h->w_gate;
    g.A1 = h->w_up;
    g.nmat = 2;
    g.nrows = c.d_ff;
    g.lda = c.d_model;
    g.K = c.d_model;
    g.B = x;
    g.ldb = c.d_model;
    e.kind = EPI_WINA;
    e.colnorm = h->ws.colnorm;
    e.s_buf = h->ws.wina_s;
    e.h_buf = h->ws.wina_h;
    hipError_t err;
    Sgemv1Desc sd = sg_base(h, bias, bias_scalar, tau);
    sd.N = c.d_ff;
    sd.K = c.d_model;
    sd.A = reinterpret_cast<const uint16_t*>(h->w_up);
    sd.vec = reinterpret_cast<const uint16_t*>(x);
    sd.Ag = reinterpret_cast<const uint16_t*>(h->w_gate);
    sd.Kg = c.d_model;
    sd.epi = SG_SCORE;
    sd.colnorm = h->ws.colnorm;
    sd.s_buf = h->ws.wina_s;
    sd.h_buf = h->ws.wina_h;
    sd.g_debug = g_debug;
    sd.s_debug = s_debug;
    if (one_token_stream(h, m, nullptr, nullptr) && sgemv1_plan(sd, h->cus)) {
      // one token: gate and up rows in one stream, the score epilogue per row
      Timed tm(h, FFN_K_GATE, s);
      err = launch_sgemv1(sd, s);
    } else {
      if (!plan_plain(g, h)) return FFN_E_UNSUPPORTED;
      Timed tm(h, FFN_K_GATE, s);
      err = launch_gemm(g, e, s);
    }
    if (err != hipSuccess) return FFN_E_HIP;
    TopkDesc td{};
    td.M = m;
    td.F = c.d_ff;
    td.k = k;
    td.T = c.tile_w;
    td.dtype = c.dtype;
    td.s_buf = h->ws.wina_s;
    td.h_buf = h->ws.wina_h;
    td.cnt = pack->cnt;
    td.idx = pack->idx;
    td.val = pack->val;
    td.route = pack->route;
    td.dense_list = pack->dense_list;
    td.n_dense = pack->n_dense;
    if (topk_out == 1) {
      td.ul_nrn = h->ws.ul_nrn;
      td.ul_hT = reinterpret_cast<uint16_t*>(h->ws.ul_h);
      td.ul_total = h->ws.ul_total;
    } else if (topk_out == 2) {
      td.hmask = h->ws.hbuf;
      td.ldhm = c.d_ff;
    }
    *routed_by_topk = true;
    Timed tm(h, FFN_K_TOPK, s);
    return hip_status(launch_topk(td, s));
  }
  if (c.in_keep > 0) {
    // input-side gate: the kept channels, then their rows of W^T in channel
    // groups; a full gate is selected and packed from the group sums, a
    // low-rank gate sums the groups into t and continues with U t
    InDesc in{};
    in.M = m;
    in.d = c.d_model;
    in.k = c.in_keep;
    in.N = c.rank ? c.rank : c.d_ff;
    in.groups = h->ws.in_groups;
    in.x = x;
    in.colnorm = h->ws.in_norm;
    in.kidx = h->ws.in_kidx;
    in.kval = h->ws.in_kval;
    in.wt = h->ws.in_wt;
    in.part = h->ws.in_part;
    in.T = c.tile_w;
    in.E = c.ell_w;
    in.sel = c.sel;
    in.bias = bias;
    in.bias_scalar = bias_scalar;
    in.tau = tau;
    in.cnt = pack->cnt;
    in.idx = pack->idx;
    in.val = pack->val;
    in.g_debug = g_debug;
    {
      Timed tm(h, FFN_K_LOWRANK_V, s);
      if (launch_in_select(in, s) != hipSuccess) return FFN_E_HIP;
    }
    {
      Timed tm(h, FFN_K_LOWRANK_V, s);
      if (launch_in_gemv(in, s) != hipSuccess) return FFN_E_HIP;
    }
    if (c.rank == 0) {
      Timed tm(h, FFN_K_GATE, s);
      return hip_status(launch_in_pack(in, s));
    }
    {
      Timed tm(h, FFN_K_LOWRANK_V, s);
      if (launch_in_sum(in, s) != hipSuccess) return FFN_E_HIP;
    }
    g.A0 = h->u;
    g.lda = c.rank;
    g.B = h->ws.in_part;                                 // t [m x rank], fp32
    g.ldb = c.rank;
    g.K = c.rank;
    g.bmode = B_F32_SPLIT;
    g.b_nsum = 1;
    g.b_slab = (long long)m * c.rank;
    e.t_out = h->ws.lr_t;
  } else if (c.rank > 0) {
    hipError_t err = hipSuccess;
    int nslabs = run_lowrank_v(h, x, m, nullptr, nullptr, s, &err);
    if (err != hipSuccess) return FFN_E_HIP;
    nslabs = collapse_slabs(h, m, nslabs, s, &err);
    if (err != hipSuccess) return FFN_E_HIP;
    g.A0 = h->u;
    g.lda = c.rank;
    b_from_slabs(g, h, nslabs);
    e.t_out = h->ws.lr_t;
  } else {
    g.A0 = h->w_gate;
    g.lda = c.d_model;
    g.K = c.d_model;
    g.B = x;
    g.ldb = c.d_model;
  }
  g.nrows = c.d_ff;
  if (!plan_twell(g, h)) return FFN_E_UNSUPPORTED;
  e.kind = EPI_TWELL;
  Timed tm(h, FFN_K_GATE, s);
  return hip_status(launch_gemm(g, e, s));
}

// Decode path (k_decode.hip) for bf16 bias / threshold configs at 1..16
// tokens: gate workgroups of R rows (16 waves for one token, 8 otherwise; R =
// waves * IPW / P on the VALU, P = pieces of 512 elements per gate row, or 32
// rows on matrix cores; R divides the TwELL tile), then the partial-row,
// chunk or split organisation of the up and down products.
bool plan_decode(const ffn_sparse_handle* h, int m, DecodeDesc* out) {
  const auto& c = h->cfg;
  if (c.dtype != FFN_BF16 || c.sel == FFN_SEL_TOPK_WINA || m < 1 || m > kDecMaxM) return false;
  if (h->tune.no_decode || c.in_keep > 0) return false;
  DecodeDesc d{};
  d.M = m;
  d.d = c.d_model;
  d.F = c.d_ff;
  d.T = c.tile_w;
  d.E = c.ell_w;
  d.rank = c.rank;
  d.K = c.rank ? c.rank : c.d_model;
  d.sel = c.sel;
  d.R = dec_gate_rows(d.K, c.tile_w, m, c.rank > 0, &d.ipw, h->tune.dec_ipw);   // at most 64 sub-tiles per TwELL tile
  // a forced piece count may give more partial rows than the workspace holds
  // (it is sized for the default shapes): then the default shape
  if (d.R && h->tune.dec_ipw && (size_t)(d.F / d.R) * std::min(m, 8) > h->ws.dec_part_rows)
    d.R = dec_gate_rows(d.K, c.tile_w, m, c.rank > 0, &d.ipw);
  if (d.R == 0 || d.F / d.R > 2048) return false;
  d.a_gate = c.rank ? h->u : h->w_gate;
  d.v = h->v;
  d.w_up = h->w_up;
  d.w_down_nm = h->w_down_nm;
  d.t = h->ws.lr_t;
  d.lb = h->ws.dec_lb;
  d.ctrl = h->ws.ctrl;
  d.umask = h->ws.umask;
  d.hd = h->ws.hd;
  d.part = h->ws.dec_part;
  d.ad = h->ws.hd;
  d.ul_total = h->ws.ul_total;
  d.ul_nrn = h->ws.ul_nrn;
  d.ul_h = h->ws.ul_h;
  d.ngroups = dec_down2_groups(d.d, d.F);
  d.nslab = c.rank ? dec_lowrank_slabs(m, c.d_model, c.rank, h->tune.lr_slabs) : 0;
  d.tslab = h->ws.lr_slabs;
  d.ldh = (d.F + 31) / 32 * 32;
  // partial rows cost M x d x 4 bytes per sub-tile: they pay off for one
  // token; from two tokens the split sequence (union list dealt evenly over
  // the chip, up and down products on matrix cores) is faster than the
  // column-chunk kernel, whose scattered loads grow with the union
  d.mode = m == 1 ? DEC_PART : DEC_SPLIT;
  if (h->tune.dec_mode >= 1 && h->tune.dec_mode <= 3 && m <= 8) d.mode = h->tune.dec_mode - 1;
  if (d.mode == DEC_SPLIT && !dec_split_ok(d)) d.mode = DEC_CHUNK;
  // 9..16 tokens: the split sequence only, with the matrix-core first stage
  if (m > 8 && (d.mode != DEC_SPLIT || (c.rank && d.nslab == 0))) return false;
  // LDS of the gate pass with hidden values (the larger of the two passes)
  const size_t stat = 8 * 1024;    // static LDS of the decode kernels, upper bound
  DecodeDesc dl = d;
  dl.up = 1;
  if (dec_gate_lds(dl) + stat > (size_t)h->lds_max) return false;
  if (c.rank && d.nslab == 0 && dec_lowrank_lds(d) + stat > (size_t)h->lds_max) return false;
  *out = d;
  return true;
}

// Gate pass of the decode path: t = V x (low rank), then the gate kernel
// (pack; with `up`, also the hidden list).
ffn_status run_dec_gate(ffn_sparse_handle* h, DecodeDesc& d, const void* x, const float* bias, float bias_scalar,
                        const float* tau, ffn_twell_pack* pack, float* g_debug, bool up, hipStream_t s) {
  d.x = x;
  d.bias = bias;
  d.bias_scalar = bias_scalar;
  d.tau = tau;
  d.cnt = pack->cnt;
  d.idx = pack->idx;
  d.val = pack->val;
  d.g_debug = g_debug;
  d.up = up ? 1 : 0;
  hipError_t err = hipSuccess;
  if (d.rank) {
    Timed tm(h, FFN_K_LOWRANK_V, s);
    err = launch_dec_lowrank(d, s);
  }
  if (err != hipSuccess) return FFN_E_HIP;
  Timed tm(h, FFN_K_GATE, s);
  return hip_status(launch_dec_gate(d, s));
}

// Launch shape of the sparse kernel: (token, group of G tiles, phase s of S)
// workgroups of 8 waves; about two workgroups per CU at most, G bounded by the
// entries a workgroup holds in LDS (a routed token evaluated here can bring T
// entries per tile), partial rows bounded by the workspace.
UpdownDesc updown_desc(const ffn_sparse_handle* h, const void* x, int m, const ffn_twell_pack* p, void* y,
                       bool include_routed) {
  const auto& c = h->cfg;
  UpdownDesc u{};
  u.dtype = c.dtype;
  u.M = m;
  u.d = c.d_model;
  u.F = c.d_ff;
  u.T = c.tile_w;
  u.E = c.ell_w;
  u.down_only = c.sel == FFN_SEL_TOPK_WINA;
  u.x = x;
  u.w_up = h->w_up;
  u.w_down_nm = h->w_down_nm;
  u.cnt = p->cnt;
  u.idx = p->idx;
  u.val = p->val;
  u.y = y;
  u.partial = h->ws.ud_partial;
  u.include_routed = include_routed ? 1 : 0;
  const int ntiles = c.d_ff / c.tile_w;
  const int per_tile = std::max(1, include_routed ? std::max(c.ell_w, c.tile_w) : c.ell_w);
  const int gcap = std::max(1, std::min(std::min(ntiles, 64), kUpdownCap / per_tile));
  const long long units = (long long)m * ntiles;
  int G = 1, S = 1;
  if (units > 2LL * h->cus) {
    // Tiles per group: the workgroups should fit two per CU (a third round on
    // some CUs cost 24 tokens at the LoPA shape 108.6 against 93.2 us). With
    // one phase, workgroup b = token * groups + group runs on XCD b mod 8, so a
    // group count that is a multiple of 8 keeps each group's weight rows on
    // one XCD's L2: that grouping is taken when it still gives 1.5 workgroups
    // per CU (56 tokens: 137 against 181 us), else the finest grouping that
    // fits (40 tokens: 118 against 134 us).
    auto groups = [&](int g) { return (long long)((ntiles + g - 1) / g); };
    int aligned = 0, fit = 0;
    for (int g = 1; g <= gcap; ++g) {
      const long long wg = (long long)m * groups(g);
      if (!fit && wg <= 2LL * h->cus) fit = g;
      if (!aligned && groups(g) % 8 == 0 && wg <= 2LL * h->cus) aligned = g;
    }
    // Beyond two workgroups per CU, eight groups (one per XCD) still win up to
    // three per CU, against the finest fitting grouping whose groups spread
    // over every XCD (LoPA, 72 tokens: 281 against 320 us, 96 tokens: 299
    // against 380 us; at 112 and 128 tokens four groups, which fit, are faster)
    const int g8 = (ntiles + 7) / 8;
    if (aligned && (long long)m * groups(aligned) * 2 >= 3LL * h->cus) G = aligned;
    else if (!aligned && g8 <= gcap && groups(g8) == 8 && 8LL * m <= 3LL * h->cus && 16LL * m >= 3LL * h->cus) G = g8;
    else G = fit ? fit : gcap;
  }
  if (h->tune.ud_group > 0) G = std::min(gcap, h->tune.ud_group);
  if (h->tune.ud_split > 0) S = std::min(16, h->tune.ud_split);
  const int epc = c.dtype == FFN_BF16 ? 8 : 4;
  u.nwaves = (h->tune.ud_waves == 4 && c.d_model / epc <= 4 * 64) ? 4 : 8;
  auto nparts = [&]() { return (long long)((ntiles + G - 1) / G) * S; };
  while (nparts() > 1 && (size_t)(m * nparts()) > h->ws.ud_rows) {
    if (S > 1) S /= 2;
    else if (G < gcap) G = std::min(gcap, G * 2);
    else break;
  }
  u.tiles_per_group = G;
  u.slot_split = S;
  // group-major within each XCD class where the grouping allows it (LoPA, 32
  // tokens: 84 against 92 us token-major; even at 48 and 64 tokens)
  u.xcd_major = (h->tune.ud_order != 1 && S == 1 && ud_groups(u) % 8 == 0) ? 1 : 0;
  u.w_gate = h->w_gate;
  u.u_rows = h->u;
  u.lr_t = h->ws.lr_t;
  u.rank = c.rank;
  u.sel = c.sel;
  return u;
}

// The XCD-sliced pair at prefill token counts (bf16 ReLU packs, routed tokens
// left to the dense backup); false when it does not apply.
static bool xcd_desc(const ffn_sparse_handle* h, const UpdownDesc& u, XcdDesc* out) {
  if (u.M < 128 || u.include_routed || u.down_only || u.dtype != DT_BF16 || h->tune.no_xcd || u.M > h->cfg.max_m)
    return false;
  XcdDesc x{};
  x.M = u.M;
  x.d = u.d;
  x.T = u.T;
  x.E = u.E;
  x.ntiles = u.F / u.T;
  x.lg_e = 0;
  while ((1 << x.lg_e) < u.E) ++x.lg_e;
  x.x = u.x;
  x.w_up = u.w_up;
  x.w_down_nm = u.w_down_nm;
  x.cnt = u.cnt;
  x.idx = u.idx;
  x.val = u.val;
  x.hp = h->ws.xh;
  x.y = u.y;
  x.route_pass = u.route_pass;
  x.route = u.route;
  if (!xcd_ok(x)) return false;
  *out = x;
  return true;
}

ffn_status run_updown(ffn_sparse_handle* h, UpdownDesc& u, hipStream_t s) {
  XcdDesc xd;
  if (xcd_desc(h, u, &xd)) {
    {
      Timed tm(h, FFN_K_UP, s);
      if (launch_xcd_up(xd, s) != hipSuccess) return FFN_E_HIP;
    }
    Timed tm(h, FFN_K_UPDOWN, s);
    return hip_status(launch_xcd_down(xd, s));
  }
  const long long nparts = (long long)ud_groups(u) * u.slot_split;
  if (nparts > 1 && (size_t)(u.M * nparts) > h->ws.ud_rows) return FFN_E_UNSUPPORTED;
  hipError_t err;
  {
    Timed tm(h, FFN_K_UPDOWN, s);
    err = launch_updown(u, s);
  }
  if (err != hipSuccess) return FFN_E_HIP;
  if (ud_groups(u) * u.slot_split == 1) return FFN_OK;
  Timed tm(h, FFN_K_REDUCE, s);
  return hip_status(launch_updown_reduce(u, s));
}

// Runs one call on a handle: refused while the handle is marked failed; a
// launch failure part-way through a call marks it.
template <typename Fn>
ffn_status guarded(ffn_sparse_handle* h, Fn fn) {
  if (h && h->failed) return FFN_E_HIP;
  const ffn_status st = fn();
  if (st == FFN_E_HIP && h) h->failed = true;
  return st;
}

}  // namespace

namespace ffn {
hipError_t dense_rows_bf16(const void* A, int nrows, int K, const void* x, int m, void* y, int ldy, int cus,
                           hipStream_t s) {
  return dense_rows_impl(A, nrows, K, x, m, y, ldy, cus, s);
}
}  // namespace ffn

extern "C" {

int32_t ffn_sparse_abi_version(void) { return FFN_SPARSE_ABI_VERSION; }

const char* ffn_sparse_status_string(ffn_status s) {
  switch (s) {
    case FFN_OK: return "ok";
    case FFN_E_INVALID: return "invalid argument";
    case FFN_E_UNSUPPORTED: return "unsupported configuration";
    case FFN_E_WORKSPACE: return "workspace too small";
    case FFN_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

ffn_status ffn_sparse_check_config(const ffn_sparse_config* c) {
  if (!c) return FFN_E_INVALID;
  if (c->dtype != FFN_F32 && c->dtype != FFN_BF16) return FFN_E_INVALID;
  if (c->act != FFN_RELU && c->act != FFN_SILU) return FFN_E_INVALID;
  if (c->sel < FFN_SEL_BIAS || c->sel > FFN_SEL_TOPK_WINA) return FFN_E_INVALID;
  if (c->wdown_out_major != 0 && c->wdown_out_major != 1) return FFN_E_INVALID;
  if (c->d_model <= 0 || c->d_ff <= 0 || c->rank < 0 || c->max_m < 1) return FFN_E_INVALID;
  if (c->tile_w <= 0 || c->ell_w < 0 || c->ell_w > c->tile_w) return FFN_E_INVALID;
  if (c->d_ff % c->tile_w != 0) return FFN_E_INVALID;
  if (c->d_model % 64 != 0) return FFN_E_UNSUPPORTED;
  if (c->d_model > (c->dtype == FFN_BF16 ? 4096 : 2048)) return FFN_E_UNSUPPORTED;
  if (c->tile_w % 16 != 0 || c->tile_w > 1024) return FFN_E_UNSUPPORTED;
  if (c->rank % 32 != 0 || c->rank > 4096) return FFN_E_UNSUPPORTED;
  if (c->max_m > 65535 || (long long)c->d_ff * c->max_m > (1ll << 31)) return FFN_E_UNSUPPORTED;
  if (c->sel != FFN_SEL_TOPK_WINA && c->act != FFN_RELU) return FFN_E_UNSUPPORTED;
  if (c->sel == FFN_SEL_TOPK_WINA && (c->ell_w != c->tile_w || c->d_ff > 32768 || c->rank != 0))
    return FFN_E_UNSUPPORTED;
  if (c->d_ff / c->tile_w > 1024) return FFN_E_UNSUPPORTED;
  if (c->in_keep < 0 || c->in_keep > c->d_model) return FFN_E_INVALID;
  // input-side gate selection: bf16, bias / threshold, no routing (the dense
  // backup would read every input channel), decode-sized batches
  if (c->in_keep > 0 && (c->dtype != FFN_BF16 || c->sel == FFN_SEL_TOPK_WINA || c->ell_w != c->tile_w ||
                         c->max_m > 64 || c->tile_w % 64 != 0))
    return FFN_E_UNSUPPORTED;
  return FFN_OK;
}

size_t ffn_sparse_workspace_bytes(const ffn_sparse_config* c) {
  if (ffn_sparse_check_config(c) != FFN_OK) return 0;
  return carve(*c, nullptr, device_cus()).total;
}

size_t ffn_sparse_pack_bytes(const ffn_sparse_config* c, int32_t m) {
  if (ffn_sparse_check_config(c) != FFN_OK || m < 0) return 0;
  const size_t nt = c->d_ff / c->tile_w, E = c->ell_w, es = esize_of(c->dtype);
  return align_up(m * nt * 4) + align_up(m * nt * E * 2) + align_up(m * nt * E * es) + align_up(m) +
         align_up(m * 4) + align_up(4);
}

ffn_status ffn_sparse_init(const ffn_sparse_config* cfg, const void* w_gate_or_u, const void* v_or_null,
                           const void* w_up, const void* w_down, void* workspace, size_t ws_bytes,
                           void* stream, ffn_sparse_handle** out) {
  if (!out) return FFN_E_INVALID;
  *out = nullptr;
  ffn_status st = ffn_sparse_check_config(cfg);
  if (st != FFN_OK) return st;
  if (!w_gate_or_u || !w_up || !w_down || !workspace) return FFN_E_INVALID;
  if (cfg->rank > 0 && !v_or_null) return FFN_E_INVALID;
  if (!aligned16(w_gate_or_u) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(workspace) ||
      (v_or_null && !aligned16(v_or_null)))
    return FFN_E_INVALID;
  const int cus = device_cus();
  Workspace ws = carve(*cfg, reinterpret_cast<char*>(workspace), cus);
  if (ws_bytes < ws.total) return FFN_E_WORKSPACE;
  {
    // the no-allocation variant's scratch on this device (set up once)
    void* scr = nullptr;
    if (scratch_for_device(reinterpret_cast<hipStream_t>(stream), &scr) != hipSuccess) return FFN_E_HIP;
  }
  ffn_sparse_handle* h = new (std::nothrow) ffn_sparse_handle();
  if (!h) return FFN_E_INVALID;
  h->cfg = *cfg;
  h->ws = ws;
  h->cus = cus;
  h->lds_max = device_lds_max();
  h->tune.no_decode = env_int("FFN_SPARSE_NO_DECODE");
  h->tune.dec_mode = env_int("FFN_SPARSE_DEC_MODE");
  h->tune.no_pf = env_int("FFN_SPARSE_NO_PREFILL_GEMM");
  h->tune.no_topk_down = env_int("FFN_SPARSE_NO_TOPK_DOWN");
  h->tune.no_xcd = env_int("FFN_SPARSE_NO_XCD");
  h->tune.no_masked_dense = env_int("FFN_SPARSE_NO_MASKED_DENSE");
#ifdef FFN_SPARSE_TUNING
  h->tune.gate_nt = env_int("FFN_SPARSE_GATE_NT");
  h->tune.gate_waves = env_int("FFN_SPARSE_GATE_WAVES");
  h->tune.ud_split = env_int("FFN_SPARSE_UD_SPLIT");
  h->tune.ud_group = env_int("FFN_SPARSE_UD_GROUP");
  h->tune.v_ks = env_int("FFN_SPARSE_V_KS");
  h->tune.no_gemv = env_int("FFN_SPARSE_NO_GEMV");
  h->tune.ud_waves = env_int("FFN_SPARSE_UD_WAVES");
  h->tune.lr_slabs = env_int("FFN_SPARSE_LR_SLABS");
  h->tune.dec_ipw = env_int("FFN_SPARSE_DEC_IPW");
  h->tune.ud_order = env_int("FFN_SPARSE_UD_ORDER");
#endif
  if (cfg->rank > 0) {
    h->u = w_gate_or_u;
    h->v = v_or_null;
  } else {
    h->w_gate = w_gate_or_u;
  }
  h->w_up = w_up;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int es = esize_of(cfg->dtype);
  hipError_t err;
  if (cfg->wdown_out_major) {
    h->w_down_om = w_down;
    h->w_down_nm = ws.wdown_alt;
    err = launch_transpose(w_down, ws.wdown_alt, cfg->d_model, cfg->d_ff, es, s);
  } else {
    h->w_down_nm = w_down;
    h->w_down_om = ws.wdown_alt;
    err = launch_transpose(w_down, ws.wdown_alt, cfg->d_ff, cfg->d_model, es, s);
  }
  if (err == hipSuccess && cfg->sel == FFN_SEL_TOPK_WINA)
    err = launch_rownorm(h->w_down_nm, ws.colnorm, cfg->d_ff, cfg->d_model, cfg->dtype, s);
  if (err == hipSuccess && cfg->in_keep > 0) {
    // the gate's input matrix input-major, and its column norms
    const int N = cfg->rank ? cfg->rank : cfg->d_ff;
    err = launch_transpose(cfg->rank ? v_or_null : w_gate_or_u, ws.in_wt, N, cfg->d_model, 2, s);
    if (err == hipSuccess) err = launch_rownorm(ws.in_wt, ws.in_norm, cfg->d_model, N, cfg->dtype, s);
  }
  if (err == hipSuccess) err = launch_fill_u32(ws.ctrl, 0u, kCtrlWords + kTicketWords, s);
  if (err == hipSuccess) err = launch_fill_u32(ws.ctrl + CTRL_SPIN_LIMIT, kDefaultSpinLimit, 1, s);
  if (err == hipSuccess)
    err = launch_fill_u32(reinterpret_cast<uint32_t*>(ws.lb), 0u,
                          (size_t)cfg->max_m * (cfg->d_ff / 16) * 2, s);
  if (err == hipSuccess)
    err = launch_fill_u32(reinterpret_cast<uint32_t*>(ws.dec_lb), 0u, (size_t)kDecMaxM * (cfg->d_ff / 2) * 2, s);
  // the split-mode list is read past its length (masked): keep its ids valid
  if (err == hipSuccess) err = launch_fill_u32(reinterpret_cast<uint32_t*>(ws.ul_nrn), 0u, cfg->d_ff, s);
  if (err == hipSuccess) err = launch_fill_u32(reinterpret_cast<uint32_t*>(ws.ul_total), 0u, 1, s);
  if (err != hipSuccess) {
    delete h;
    return FFN_E_HIP;
  }
  *out = h;
  return FFN_OK;
}

static ffn_status gate_pack_impl(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                float bias_scalar, const float* tau, int32_t k, ffn_twell_pack* pack,
                                float* g_debug, float* s_debug, void* stream) {
  ffn_status st = check_call(h, x, m, tau, k);
  if (st != FFN_OK) return st;
  if (!pack_ok(pack)) return FFN_E_INVALID;
  if (s_debug && h->cfg.sel != FFN_SEL_TOPK_WINA) return FFN_E_INVALID;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (m == 0) return hip_status(launch_fill_u32(reinterpret_cast<uint32_t*>(pack->n_dense), 0u, 1, s));
  bool routed_by_topk = false;
  DecodeDesc dd;
  if (plan_decode(h, m, &dd)) st = run_dec_gate(h, dd, x, bias, bias_scalar, tau, pack, g_debug, false, s);
  else st = gate_pack_core(h, x, m, bias, bias_scalar, tau, k, pack, g_debug, s_debug, s, &routed_by_topk);
  if (st != FFN_OK || routed_by_topk) return st;
  Timed tm(h, FFN_K_ROUTE, s);
  return hip_status(launch_route(route_desc(h, m, pack), s));
}

static ffn_status updown_impl(ffn_sparse_handle* h, const void* x, int32_t m, const ffn_twell_pack* pack,
                             void* y, void* stream) {
  ffn_status st = check_call(h, x, m, reinterpret_cast<const float*>(1), 0);
  if (st != FFN_OK) return st;
  if (!pack_ok(pack) || (m > 0 && (!y || !aligned16(y)))) return FFN_E_INVALID;
  if (m == 0) return FFN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  UpdownDesc u = updown_desc(h, x, m, pack, y, false);
  return run_updown(h, u, s);
}

static ffn_status dense_fallback_impl(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                     float bias_scalar, const float* tau, int32_t k,
                                     const ffn_twell_pack* pack, void* y, void* stream) {
  ffn_status st = check_call(h, x, m, tau, k);
  if (st != FFN_OK) return st;
  if (!pack_ok(pack) || (m > 0 && (!y || !aligned16(y)))) return FFN_E_INVALID;
  const auto& c = h->cfg;
  // a top-k pack has E == T: no tile can overflow, nothing is ever routed
  if (m == 0 || c.sel == FFN_SEL_TOPK_WINA || c.ell_w >= c.tile_w) return FFN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = run_dense_hidden(h, x, m, pack->dense_list, pack->n_dense, bias, bias_scalar, tau,
                                    FFN_K_FALLBACK, s);
  if (err != hipSuccess) return FFN_E_HIP;
  return hip_status(run_dense_down(h, m, pack->dense_list, pack->n_dense, y, FFN_K_FALLBACK, s));
}

// Descriptor of the list-driven down kernel for one token's top-k list
// (written by the top-k kernel); false when the shape does not fit it.
static bool topk_list_desc(const ffn_sparse_handle* h, void* y, DecodeDesc* out) {
  const auto& c = h->cfg;
  DecodeDesc d{};
  d.M = 1;
  d.d = c.d_model;
  d.F = c.d_ff;
  d.T = c.tile_w;
  d.R = 64;
  d.w_down_nm = h->w_down_nm;
  d.ul_total = h->ws.ul_total;
  d.ul_nrn = h->ws.ul_nrn;
  d.ul_h = h->ws.ul_h;
  d.ldh = (d.F + 31) / 32 * 32;
  d.ngroups = dec_down2_groups(d.d, d.F);
  d.part = h->ws.dec_part;
  d.y = y;
  d.route_pass = 0;                    // the top-k kernel has routed the pack
  if (!dec_split_ok(d)) return false;
  *out = d;
  return true;
}

// Down-product organisation of top-k selection's forward pass: 0 the
// per-token TwELL kernel (fp32, or forced by the tuning switch), 1 the
// one-token list kernel, 2 the dense product of masked h rows.
static int topk_down_kind(const ffn_sparse_handle* h, int m) {
  const auto& c = h->cfg;
  if (c.sel != FFN_SEL_TOPK_WINA || c.dtype != FFN_BF16 || h->tune.no_topk_down || m < 1) return 0;
  DecodeDesc ld;
  return (m == 1 && topk_list_desc(h, nullptr, &ld)) ? 1 : 2;
}

// The masked dense sequence (bf16 bias / threshold selection, 17..127
// tokens): the dense hidden activations h = a(z) * (W_up x) with the
// selection applied to every neuron, the gate values kept in g_ext; the TwELL
// pack built from those same gate values (so the pack and y take the same
// decisions); the route pass; a dense down GEMM. Every token is evaluated this
// way, routed or not.
static bool masked_dense_ok(const ffn_sparse_handle* h, int m) {
  const auto& c = h->cfg;
  return c.dtype == FFN_BF16 && c.sel != FFN_SEL_TOPK_WINA && c.in_keep == 0 && !h->tune.no_masked_dense &&
         m > kDecMaxM && m <= masked_dense_max_m(c) && m <= c.max_m;
}

static ffn_status masked_dense_forward(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                       float bias_scalar, const float* tau, ffn_twell_pack* pack, void* y,
                                       hipStream_t s) {
  const auto& c = h->cfg;
  if (run_dense_hidden(h, x, m, nullptr, nullptr, bias, bias_scalar, tau, FFN_K_UP, s, true, FFN_K_GATE) !=
      hipSuccess)
    return FFN_E_HIP;
  PackGDesc pd{};
  pd.M = m;
  pd.F = c.d_ff;
  pd.T = c.tile_w;
  pd.E = c.ell_w;
  pd.sel = c.sel;
  pd.out_f32 = 0;
  pd.g = h->ws.g_ext;
  pd.bias = bias;
  pd.bias_scalar = bias_scalar;
  pd.tau = tau;
  pd.cnt = pack->cnt;
  pd.idx = pack->idx;
  pd.val = pack->val;
  {
    Timed tm(h, FFN_K_ROUTE, s);
    if (launch_pack_g(pd, s) != hipSuccess) return FFN_E_HIP;
  }
  {
    Timed tm(h, FFN_K_ROUTE, s);
    if (launch_route(route_desc(h, m, pack), s) != hipSuccess) return FFN_E_HIP;
  }
  return hip_status(run_dense_down(h, m, nullptr, nullptr, y, FFN_K_UPDOWN, s));
}

static ffn_status forward_impl(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                              float bias_scalar, const float* tau, int32_t k, ffn_twell_pack* pack,
                              void* y, void* stream) {
  ffn_status st = check_call(h, x, m, tau, k);
  if (st != FFN_OK) return st;
  if (!pack_ok(pack) || (m > 0 && (!y || !aligned16(y)))) return FFN_E_INVALID;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (m == 0) return hip_status(launch_fill_u32(reinterpret_cast<uint32_t*>(pack->n_dense), 0u, 1, s));
  DecodeDesc dd;
  if (plan_decode(h, m, &dd)) {
    st = run_dec_gate(h, dd, x, bias, bias_scalar, tau, pack, nullptr, true, s);
    if (st != FFN_OK) return st;
    dd.y = y;
    dd.route_pass = 1;
    dd.route = route_desc(h, m, pack);
    if (dd.mode == DEC_SPLIT) {
      Timed tu(h, FFN_K_UP, s);
      if (launch_dec_up(dd, s) != hipSuccess) return FFN_E_HIP;
    }
    Timed tm(h, FFN_K_UPDOWN, s);
    if (dd.mode == DEC_PART) return hip_status(launch_dec_reduce(dd, s));
    if (dd.mode == DEC_SPLIT) return hip_status(launch_dec_down2(dd, s));
    return hip_status(launch_dec_down(dd, s));
  }
  if (masked_dense_ok(h, m)) return masked_dense_forward(h, x, m, bias, bias_scalar, tau, pack, y, s);
  const auto& c = h->cfg;
  // top-k selection keeps a fixed share of every token's neurons: one token's
  // kept rows go to the list-driven down kernel; from two tokens the union of
  // the kept sets covers most of W_down, so the masked h rows go to a dense
  // down product
  const int topk_out = topk_down_kind(h, m);
  DecodeDesc ld{};
  if (topk_out == 1 && !topk_list_desc(h, y, &ld)) return FFN_E_UNSUPPORTED;
  bool routed_by_topk = false;
  st = gate_pack_core(h, x, m, bias, bias_scalar, tau, k, pack, nullptr, nullptr, s, &routed_by_topk, topk_out);
  if (st != FFN_OK) return st;
  if (topk_out == 1) {
    Timed tm(h, FFN_K_UPDOWN, s);
    return hip_status(launch_dec_down2(ld, s));
  }
  if (topk_out == 2) return hip_status(run_dense_down(h, m, nullptr, nullptr, y, FFN_K_UPDOWN, s));
  const bool can_route = c.sel != FFN_SEL_TOPK_WINA && c.ell_w < c.tile_w;
  const bool decode = m <= kDecodeMaxM;
  UpdownDesc u = updown_desc(h, x, m, pack, y, decode && can_route);
  u.route_pass = routed_by_topk ? 0 : 1;          // block 0 routes the pack (top-k already did)
  u.route = route_desc(h, m, pack);
  u.bias = bias;
  u.bias_scalar = bias_scalar;
  u.tau = tau;
  st = run_updown(h, u, s);
  if (st != FFN_OK || decode || !can_route) return st;
  hipError_t err = run_dense_hidden(h, x, m, pack->dense_list, pack->n_dense, bias, bias_scalar, tau,
                                    FFN_K_FALLBACK, s);
  if (err != hipSuccess) return FFN_E_HIP;
  return hip_status(run_dense_down(h, m, pack->dense_list, pack->n_dense, y, FFN_K_FALLBACK, s));
}

static ffn_status dense_forward_impl(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                    float bias_scalar, const float* tau, void* y, void* stream) {
  ffn_status st = check_call(h, x, m, tau, 0);
  if (st != FFN_OK) return st;
  if (m > 0 && (!y || !aligned16(y))) return FFN_E_INVALID;
  if (m == 0) return FFN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = run_dense_hidden(h, x, m, nullptr, nullptr, bias, bias_scalar, tau, FFN_K_DENSE, s);
  if (err != hipSuccess) return FFN_E_HIP;
  return hip_status(run_dense_down(h, m, nullptr, nullptr, y, FFN_K_DENSE, s));
}

ffn_status ffn_sparse_gate_pack(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                float bias_scalar, const float* tau, int32_t k, ffn_twell_pack* pack,
                                float* g_debug, float* s_debug, void* stream) {
  return guarded(h, [&] { return gate_pack_impl(h, x, m, bias, bias_scalar, tau, k, pack, g_debug, s_debug, stream); });
}

ffn_status ffn_sparse_updown(ffn_sparse_handle* h, const void* x, int32_t m, const ffn_twell_pack* pack,
                             void* y, void* stream) {
  return guarded(h, [&] { return updown_impl(h, x, m, pack, y, stream); });
}

ffn_status ffn_sparse_dense_fallback(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                     float bias_scalar, const float* tau, int32_t k,
                                     const ffn_twell_pack* pack, void* y, void* stream) {
  return guarded(h, [&] { return dense_fallback_impl(h, x, m, bias, bias_scalar, tau, k, pack, y, stream); });
}

ffn_status ffn_sparse_forward(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                              float bias_scalar, const float* tau, int32_t k, ffn_twell_pack* pack,
                              void* y, void* stream) {
  return guarded(h, [&] { return forward_impl(h, x, m, bias, bias_scalar, tau, k, pack, y, stream); });
}

ffn_status ffn_sparse_dense_forward(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                    float bias_scalar, const float* tau, void* y, void* stream) {
  return guarded(h, [&] { return dense_forward_impl(h, x, m, bias, bias_scalar, tau, y, stream); });
}

ffn_status ffn_sparse_forward_noalloc(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                      float bias_scalar, const float* tau, int32_t k, ffn_twell_pack* pack,
                                      void* y, void* stream) {
  return guarded(h, [&]() -> ffn_status {
    ffn_status st = check_call(h, x, m, tau, k);
    if (st != FFN_OK) return st;
    if (!pack_ok(pack) || (m > 0 && (!y || !aligned16(y)))) return FFN_E_INVALID;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (m == 0) return hip_status(launch_fill_u32(reinterpret_cast<uint32_t*>(pack->n_dense), 0u, 1, s));
    const auto& c = h->cfg;
    DecodeDesc dd;
    if (!plan_decode(h, m, &dd) || c.d_ff > kScrMaxF) return FFN_E_UNSUPPORTED;
    void* base = nullptr;
    if (scratch_for_device(s, &base) != hipSuccess) return FFN_E_HIP;
    // per-call regions after the fixed ones, sized for this call
    char* p = reinterpret_cast<char*>(base);
    size_t off = kScrFixedBytes;
    auto take = [&](size_t bytes) -> char* {
      char* q = p + off;
      off += align_up(bytes);
      return q;
    };
    const size_t F = c.d_ff, d = c.d_model, r = c.rank, M = m;
    Workspace w = h->ws;
    w.ctrl = reinterpret_cast<uint32_t*>(p);
    w.dec_lb = reinterpret_cast<uint64_t*>(p + kScrCtrlBytes);
    w.ul_nrn = reinterpret_cast<int32_t*>(p + kScrCtrlBytes + kScrLbBytes);
    w.ul_total = reinterpret_cast<int32_t*>(p + kScrCtrlBytes + kScrLbBytes + kScrIdsBytes);
    w.lr_slabs = reinterpret_cast<float*>(take(std::max<size_t>(1, 8 * M * r) * sizeof(float)));
    w.lr_t = reinterpret_cast<float*>(take(std::max<size_t>(1, M * r) * sizeof(float)));
    w.umask = reinterpret_cast<uint64_t*>(take((F / 2) * sizeof(uint64_t)));
    w.hd = reinterpret_cast<float*>(take(F * M * sizeof(float)));
    const size_t rows = dd.mode == DEC_PART ? (F / dd.R) * M : (dd.mode == DEC_SPLIT ? (size_t)dd.ngroups * M : 1);
    w.dec_part = reinterpret_cast<float*>(take(rows * d * sizeof(float)));
    w.dec_part_rows = rows;
    w.ul_h = reinterpret_cast<float*>(take(M * ((F + 31) / 32 * 32) * sizeof(uint16_t)));
    if (off > kScratchBytes) return FFN_E_WORKSPACE;
    const Workspace saved = h->ws;
    h->ws = w;
    st = forward_impl(h, x, m, bias, bias_scalar, tau, k, pack, y, stream);
    h->ws = saved;
    return st;
  });
}

size_t ffn_sparse_noalloc_scratch_bytes(void) { return kScratchBytes; }

ffn_status ffn_sparse_device_status(ffn_sparse_handle* h, void* stream) {
  if (!h) return FFN_E_INVALID;
  if (h->failed) return FFN_E_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t err = 0;
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(&err, h->ws.ctrl + CTRL_ERR, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess || err != 0 ||
      scratch_error_word() != 0) {
    h->failed = true;
    return FFN_E_HIP;
  }
  return FFN_OK;
}

ffn_status ffn_sparse_debug_waits(ffn_sparse_handle* h, uint32_t epoch_skew, uint32_t spin_limit, void* stream) {
  if (!h) return FFN_E_INVALID;
  if (h->failed) return FFN_E_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (launch_fill_u32(h->ws.ctrl + CTRL_WAIT_SKEW, epoch_skew, 1, s) != hipSuccess ||
      launch_fill_u32(h->ws.ctrl + CTRL_SPIN_LIMIT, spin_limit, 1, s) != hipSuccess) {
    h->failed = true;
    return FFN_E_HIP;
  }
  return FFN_OK;
}

int32_t ffn_sparse_forward_path(const ffn_sparse_handle* h, int32_t m) {
  if (!h || m < 0 || m > h->cfg.max_m) return -1;
  if (h->cfg.in_keep > 0) return 6;
  DecodeDesc dd;
  if (plan_decode(h, m, &dd)) return 1 + dd.mode;
  if (topk_down_kind(h, m) == 1) return 4;
  if (topk_down_kind(h, m) == 2) return 5;
  if (masked_dense_ok(h, m)) return 7;
  return 0;
}

// ------------------------------------------------------------------ backward pass
namespace {
// (the per-token input-gradient kernel lists a token's pack slots, or a routed
// token's neurons, in 8192 LDS entries)
bool bw_supported(const ffn_sparse_config& c) {
  const long long slots = (long long)(c.d_ff / c.tile_w) * c.ell_w;
  return c.rank == 0 && c.act == FFN_RELU && c.sel != FFN_SEL_TOPK_WINA && c.in_keep == 0 && c.d_model <= 4096 &&
         c.tile_w <= 1024 && slots <= 8192 && (c.ell_w >= c.tile_w || c.d_ff <= 8192);
}
// dx on matrix cores (bf16, training batch sizes): see k_bw_duz
bool bw_dx_dense(const ffn_sparse_config& c, int m) {
  return c.dtype == FFN_BF16 && m >= kBwDxDenseMin && c.d_ff % 32 == 0 && c.d_model % 64 == 0;
}
struct BwLayout {
  size_t slot, zr, blk, colptr, ent_tok, ent_pos, du, dz, dxp, wt, duz, total;
  long long pbase, pcap;
  int nblk;
};
BwLayout bw_layout(const ffn_sparse_config& c, int m) {
  BwLayout L{};
  const long long ntiles = c.d_ff / c.tile_w;
  const bool routing = c.ell_w < c.tile_w;
  L.pbase = (long long)m * ntiles * c.ell_w;
  L.pcap = L.pbase + (routing ? (long long)m * c.d_ff : 0);
  L.nblk = (m + kBwBlock - 1) / kBwBlock;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  L.slot = take((size_t)m * 4);
  L.zr = take(routing ? (size_t)m * c.d_ff * 4 : 4);
  L.blk = take((size_t)L.nblk * c.d_ff * 4);
  L.colptr = take((size_t)(c.d_ff + 1) * 4);
  L.ent_tok = take((size_t)L.pcap * 4);
  L.ent_pos = take((size_t)L.pcap * 4);
  L.du = take((size_t)L.pcap * 4);
  L.dz = take((size_t)L.pcap * 4);
  const int S = bw_dx_splits(m);
  L.dxp = take(S > 1 ? (size_t)S * m * c.d_model * 4 : 4);
  // matrix-core dx: [W_up; W_gate] transposed, [d x 2F], and the (du | dz) rows
  const bool dense_dx = bw_dx_dense(c, m);
  L.wt = take(dense_dx ? (size_t)c.d_model * 2 * c.d_ff * 2 : 4);
  L.duz = take(dense_dx ? (size_t)m * 2 * c.d_ff * 2 : 4);
  L.total = o;
  return L;
}
}  // namespace

size_t ffn_sparse_backward_workspace_bytes(const ffn_sparse_config* cfg, int32_t m) {
  if (ffn_sparse_check_config(cfg) != FFN_OK || !bw_supported(*cfg) || m < 1 || m > cfg->max_m) return 0;
  const BwLayout L = bw_layout(*cfg, m);
  if (L.pcap >= (1LL << 31)) return 0;
  return L.total;
}

ffn_status ffn_sparse_backward(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias, float bias_scalar,
                               const float* tau, const ffn_twell_pack* pack, const void* dy, void* dx,
                               float* dw_gate, float* dw_up, float* dw_down_nm, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return guarded(h, [&]() -> ffn_status {
    ffn_status st = check_call(h, x, m, tau, 0);
    if (st != FFN_OK) return st;
    const auto& c = h->cfg;
    if (!bw_supported(c)) return FFN_E_UNSUPPORTED;
    if (m == 0) return FFN_OK;
    if (!pack_ok(pack) || !dy || !aligned16(dy) || (dx && !aligned16(dx)) || (dw_gate && !aligned16(dw_gate)) ||
        (dw_up && !aligned16(dw_up)) || (dw_down_nm && !aligned16(dw_down_nm)) || !workspace ||
        !aligned16(workspace))
      return FFN_E_INVALID;
    if (workspace_bytes < ffn_sparse_backward_workspace_bytes(&c, m)) return FFN_E_WORKSPACE;
    const BwLayout L = bw_layout(c, m);
    char* w = static_cast<char*>(workspace);
    BwDesc d{};
    d.m = m;
    d.d = c.d_model;
    d.F = c.d_ff;
    d.T = c.tile_w;
    d.E = c.ell_w;
    d.ntiles = c.d_ff / c.tile_w;
    d.dtype = c.dtype == FFN_BF16 ? DT_BF16 : DT_F32;
    d.sel = c.sel;
    d.nblk = L.nblk;
    d.routing = c.ell_w < c.tile_w;
    d.x = x;
    d.dy = dy;
    d.dx = dx;
    d.w_gate = h->w_gate;
    d.w_up = h->w_up;
    d.w_down_nm = h->w_down_nm;
    d.bias = bias;
    d.bias_scalar = bias_scalar;
    d.tau = tau;
    d.cnt = pack->cnt;
    d.idx = pack->idx;
    d.val = pack->val;
    d.route = pack->route;
    d.dense_list = pack->dense_list;
    d.n_dense = pack->n_dense;
    d.slot_of = reinterpret_cast<int32_t*>(w + L.slot);
    d.zr = reinterpret_cast<float*>(w + L.zr);
    d.blk = reinterpret_cast<int32_t*>(w + L.blk);
    d.colptr = reinterpret_cast<int32_t*>(w + L.colptr);
    d.ent_tok = reinterpret_cast<int32_t*>(w + L.ent_tok);
    d.ent_pos = reinterpret_cast<int32_t*>(w + L.ent_pos);
    d.du = reinterpret_cast<float*>(w + L.du);
    d.dz = reinterpret_cast<float*>(w + L.dz);
    d.dxp = reinterpret_cast<float*>(w + L.dxp);
    d.pbase = L.pbase;
    d.dw_gate = dw_gate;
    d.dw_up = dw_up;
    d.dw_down = dw_down_nm;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = launch_bw_slots(d, s);
    if (e == hipSuccess && d.routing) {
      // the routed tokens' gate rows, densely (dense-list slot order)
      GemmDesc g = gemm_base(h);
      g.A0 = h->w_gate;
      g.nrows = c.d_ff;
      g.lda = c.d_model;
      g.K = c.d_model;
      g.B = x;
      g.ldb = c.d_model;
      g.M = m;
      g.gather = pack->dense_list;
      g.m_dev = pack->n_dense;
      EpiDesc ep = epi_base(h, nullptr, 0.f, nullptr);
      ep.kind = EPI_STORE_F32;
      ep.out = reinterpret_cast<float*>(w + L.zr);
      ep.ldo = c.d_ff;
      ep.out_slab = 0;
      if (!plan_plain(g, h) || g.ks != 1) return FFN_E_UNSUPPORTED;
      Timed tm(h, FFN_K_BW_GATE, s);
      e = launch_gemm(g, ep, s);
    }
    if (e == hipSuccess) e = launch_bw_count(d, s);
    if (e == hipSuccess) e = launch_bw_scan(d, s);
    if (e == hipSuccess) e = launch_bw_fill(d, s);
    if (e == hipSuccess) {
      Timed tm(h, FFN_K_BW_NEURON, s);
      e = launch_bw_neuron(d, s);
    }
    GemmDesc gdx = gemm_base(h);
    const bool dense_dx = dx && bw_dx_dense(c, m) && [&] {
      gdx.A0 = w + L.wt;
      gdx.nrows = c.d_model;
      gdx.lda = 2 * c.d_ff;
      gdx.K = 2 * c.d_ff;
      gdx.B = w + L.duz;
      gdx.ldb = 2 * c.d_ff;
      gdx.M = m;
      return plan_plain(gdx, h);
    }();
    if (e == hipSuccess && dx) {
      if (dense_dx) {
        // dx = (du | dz) [W_up; W_gate] on matrix cores: both weights
        // transposed side by side into [d x 2F], the dense rows, one GEMM
        uint16_t* wt = reinterpret_cast<uint16_t*>(w + L.wt);
        d.duz = reinterpret_cast<uint16_t*>(w + L.duz);
        EpiDesc ep{};
        ep.kind = EPI_Y;
        ep.F = c.d_model;
        ep.out_f32 = false;
        ep.y = dx;
        ep.ldy = c.d_model;
        // four launches, each timed under the dx role
        {
          Timed tm(h, FFN_K_BW_DX, s);
          e = launch_transpose_ld(h->w_up, wt, c.d_ff, c.d_model, 2 * c.d_ff, 2, s);
        }
        if (e == hipSuccess) {
          Timed tm(h, FFN_K_BW_DX, s);
          e = launch_transpose_ld(h->w_gate, wt + c.d_ff, c.d_ff, c.d_model, 2 * c.d_ff, 2, s);
        }
        if (e == hipSuccess) {
          Timed tm(h, FFN_K_BW_DX, s);
          e = launch_bw_duz(d, s);
        }
        if (e == hipSuccess) {
          Timed tm(h, FFN_K_BW_DX, s);
          e = launch_gemm(gdx, ep, s);
        }
      } else {
        Timed tm(h, FFN_K_BW_DX, s);
        e = launch_bw_dx(d, s);
      }
    }
    return hip_status(e);
  });
}

namespace {
// A TwELL pack for m tokens in `base` (the layout ffn_sparse_pack_bytes sizes).
ffn_twell_pack carve_pack(char* base, const ffn_sparse_config& c, int m) {
  const size_t nt = c.d_ff / c.tile_w, E = c.ell_w, es = esize_of(c.dtype);
  ffn_twell_pack p{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* q = base + o;
    o += align_up(bytes);
    return q;
  };
  p.cnt = reinterpret_cast<int32_t*>(take((size_t)m * nt * 4));
  p.idx = reinterpret_cast<uint16_t*>(take((size_t)m * nt * E * 2));
  p.val = take((size_t)m * nt * E * es);
  p.route = reinterpret_cast<uint8_t*>(take((size_t)m));
  p.dense_list = reinterpret_cast<int32_t*>(take((size_t)m * 4));
  p.n_dense = reinterpret_cast<int32_t*>(take(4));
  return p;
}
}  // namespace

size_t ffn_sparse_moe_workspace_bytes(const ffn_sparse_config* cfg, int32_t m, int32_t topk) {
  if (ffn_sparse_check_config(cfg) != FFN_OK || m < 1 || topk < 1 || (size_t)m * topk > (size_t)kMoeMaxPairs)
    return 0;
  const size_t np = (size_t)m * topk, rowb = (size_t)cfg->d_model * esize_of(cfg->dtype);
  // + the grouped experts' own packs: one single-token pack per pair covers
  // them (the pack size is subadditive in the token count)
  return 2 * align_up(np * rowb) + 2 * align_up(np * 4) + ffn_sparse_pack_bytes(cfg, m) +
         np * ffn_sparse_pack_bytes(cfg, 1);
}

ffn_status ffn_sparse_moe_forward(ffn_sparse_handle* const* experts, int32_t n_experts, const void* x, int32_t m,
                                  int32_t topk, const int32_t* expert_ids, const float* weights, const float* bias,
                                  float bias_scalar, const float* tau, int32_t k, int32_t dense, void* workspace,
                                  size_t workspace_bytes, void* y, void* stream) {
  if (!experts || n_experts < 1 || m < 0 || topk < 1 || topk > n_experts) return FFN_E_INVALID;
  for (int e = 0; e < n_experts; ++e) {
    if (!experts[e]) return FFN_E_INVALID;
    if (experts[e]->failed) return FFN_E_HIP;
    ffn_sparse_config a = experts[e]->cfg, b = experts[0]->cfg;
    a.max_m = b.max_m = 0;
    if (std::memcmp(&a, &b, sizeof(a)) != 0) return FFN_E_INVALID;    // one shape for every expert
  }
  if (m == 0) return FFN_OK;
  const auto& c = experts[0]->cfg;
  if ((size_t)m * topk > (size_t)kMoeMaxPairs || !expert_ids || !weights || !x || !y || !aligned16(x) ||
      !aligned16(y) || !workspace || !aligned16(workspace))
    return FFN_E_INVALID;
  if (c.sel == FFN_SEL_THRESH && !tau) return FFN_E_INVALID;
  if (workspace_bytes < ffn_sparse_moe_workspace_bytes(&c, m, topk)) return FFN_E_WORKSPACE;
  // routing table (host): experts' rows contiguous, tokens in order
  const int np = m * topk;
  std::vector<int> cnt(n_experts, 0), off(n_experts + 1, 0);
  for (int q = 0; q < np; ++q) {
    const int e = expert_ids[q];
    if (e < 0 || e >= n_experts || !std::isfinite(weights[q])) return FFN_E_INVALID;
    for (int s2 = 0; s2 < q % topk; ++s2)
      if (expert_ids[q - q % topk + s2] == e) return FFN_E_INVALID;     // one slot per expert and token
    ++cnt[e];
  }
  for (int e = 0; e < n_experts; ++e) {
    if (cnt[e] > experts[e]->cfg.max_m) return FFN_E_INVALID;
    off[e + 1] = off[e] + cnt[e];
  }
  MoeDesc md{};
  md.d = c.d_model;
  md.m = m;
  md.topk = topk;
  md.npairs = np;
  md.dtype = c.dtype == FFN_BF16 ? DT_BF16 : DT_F32;
  {
    std::vector<int> fill(off.begin(), off.end() - 1);
    for (int t = 0; t < m; ++t)
      for (int s2 = 0; s2 < topk; ++s2) {
        const int q = t * topk + s2, e = expert_ids[q], r = fill[e]++;
        md.tab.src[r] = q;
        md.tab.pos[q] = r;
        md.tab.w[q] = weights[q];
      }
  }
  const size_t rowb = (size_t)c.d_model * esize_of(c.dtype);
  char* p = static_cast<char*>(workspace);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* q = p + o;
    o += align_up(bytes);
    return q;
  };
  md.x = x;
  md.xg = take((size_t)np * rowb);
  md.yg = take((size_t)np * rowb);
  md.tg = reinterpret_cast<float*>(take((size_t)np * 4));
  md.bg = reinterpret_cast<float*>(take((size_t)np * 4));
  md.tau = tau;
  md.bias = bias;
  md.y = y;
  const size_t nt = c.d_ff / c.tile_w, E = c.ell_w;
  ffn_twell_pack pk{};
  pk.cnt = reinterpret_cast<int32_t*>(take((size_t)m * nt * 4));
  pk.idx = reinterpret_cast<uint16_t*>(take((size_t)m * nt * E * 2));
  pk.val = take((size_t)m * nt * E * esize_of(c.dtype));
  pk.route = reinterpret_cast<uint8_t*>(take((size_t)m));
  pk.dense_list = reinterpret_cast<int32_t*>(take((size_t)m * 4));
  pk.n_dense = reinterpret_cast<int32_t*>(take(4));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (launch_moe_gather(md, s) != hipSuccess) return FFN_E_HIP;
  // The active experts, grouped by their decode sequence: one-token experts
  // (partial rows) and 2..8-token experts (the split sequence, planned for
  // the group's largest count) run one launch per kernel for the whole group
  // (grid.y or grid.z picks the expert), each expert with its own pack; any
  // other expert runs its own sequence.
  std::vector<int> one, multi, rest;
  int mmax = 0;
  for (int e = 0; e < n_experts; ++e) {
    if (!cnt[e]) continue;
    if (dense) rest.push_back(e);
    else if (cnt[e] == 1) one.push_back(e);
    else if (cnt[e] <= 8 && c.rank > 0) {
      multi.push_back(e);
      mmax = std::max(mmax, cnt[e]);
    } else {
      rest.push_back(e);
    }
  }
  std::vector<DecodeDesc> d1(one.size()), dm(multi.size());
  bool g1 = !one.empty();
  for (size_t a = 0; a < one.size() && g1; ++a)
    g1 = plan_decode(experts[one[a]], 1, &d1[a]) && d1[a].mode == DEC_PART;
  if (!g1) rest.insert(rest.end(), one.begin(), one.end());
  bool gm = !multi.empty();
  for (size_t a = 0; a < multi.size() && gm; ++a)
    gm = experts[multi[a]]->cfg.max_m >= mmax && plan_decode(experts[multi[a]], mmax, &dm[a]) &&
         dm[a].mode == DEC_SPLIT && dec_split_group_shape(dm[a]);
  if (!gm) rest.insert(rest.end(), multi.begin(), multi.end());
  // the expert's rows, selection inputs, own pack and output rows
  auto bind = [&](DecodeDesc& d, int e) {
    const ffn_twell_pack pe = carve_pack(take(ffn_sparse_pack_bytes(&c, cnt[e])), c, cnt[e]);
    d.M = cnt[e];
    d.x = static_cast<const char*>(md.xg) + (size_t)off[e] * rowb;
    d.bias = bias ? md.bg + off[e] : nullptr;
    d.bias_scalar = bias_scalar;
    d.tau = tau ? md.tg + off[e] : nullptr;
    d.cnt = pe.cnt;
    d.idx = pe.idx;
    d.val = pe.val;
    d.g_debug = nullptr;
    d.up = 1;
    d.y = static_cast<char*>(const_cast<void*>(md.yg)) + (size_t)off[e] * rowb;
    d.route_pass = 1;
    d.route = route_desc(experts[e], cnt[e], &pe);
  };
  auto fail = [&](const std::vector<int>& ids, size_t a0, int n) {
    for (int i = 0; i < n; ++i) experts[ids[a0 + i]]->failed = true;
    return FFN_E_HIP;
  };
  if (gm) {
    for (size_t a = 0; a < multi.size(); ++a) bind(dm[a], multi[a]);
    ffn_sparse_handle* h0 = experts[multi[0]];
    for (size_t a0 = 0; a0 < multi.size(); a0 += kDecGroupMax) {
      const int n = (int)std::min<size_t>(kDecGroupMax, multi.size() - a0);
      DecGroup g{};
      for (int i = 0; i < n; ++i) g.d[i] = dm[a0 + i];
      static const int kind[4] = {FFN_K_LOWRANK_V, FFN_K_GATE, FFN_K_UP, FFN_K_UPDOWN};
      for (int stage = 0; stage < 4; ++stage) {
        Timed tm(h0, kind[stage], s);
        if (launch_dec_split_group(g, n, stage, s) != hipSuccess) return fail(multi, a0, n);
      }
    }
  }
  if (g1) {
    for (size_t a = 0; a < one.size(); ++a) bind(d1[a], one[a]);
    ffn_sparse_handle* h0 = experts[one[0]];
    for (size_t a0 = 0; a0 < one.size(); a0 += kDecGroupMax) {
      const int n = (int)std::min<size_t>(kDecGroupMax, one.size() - a0);
      DecGroup g{};
      for (int i = 0; i < n; ++i) g.d[i] = d1[a0 + i];
      hipError_t err = hipSuccess;
      if (c.rank) {
        Timed tm(h0, FFN_K_LOWRANK_V, s);
        err = launch_dec_lowrank_group(g, n, s);
      }
      if (err == hipSuccess) {
        Timed tm(h0, FFN_K_GATE, s);
        err = launch_dec_gate_group(g, n, s);
      }
      if (err == hipSuccess) {
        Timed tm(h0, FFN_K_UPDOWN, s);
        err = launch_dec_reduce_group(g, n, s);
      }
      if (err != hipSuccess) return fail(one, a0, n);
    }
  }
  // every other expert's forward pass on its rows, in expert order, with the
  // shared pack
  std::sort(rest.begin(), rest.end());
  for (const int e : rest) {
    const char* xe = static_cast<const char*>(md.xg) + (size_t)off[e] * rowb;
    void* ye = static_cast<char*>(const_cast<void*>(md.yg)) + (size_t)off[e] * rowb;
    const float* be = bias ? md.bg + off[e] : nullptr;
    const float* te = tau ? md.tg + off[e] : nullptr;
    const ffn_status st = dense ? ffn_sparse_dense_forward(experts[e], xe, cnt[e], be, bias_scalar, te, ye, stream)
                                : ffn_sparse_forward(experts[e], xe, cnt[e], be, bias_scalar, te, k, &pk, ye, stream);
    if (st != FFN_OK) return st;
  }
  return hip_status(launch_moe_combine(md, s));
}

ffn_status ffn_sparse_timing_enable(ffn_sparse_handle* h, int32_t enable, int32_t capacity) {
  if (!h || capacity < 0) return FFN_E_INVALID;
  if (!enable) {
    h->timing = false;
    return FFN_OK;
  }
  if (capacity > h->cap) {
    for (int k = 0; k < FFN_K_COUNT; ++k)
      for (int w = 0; w < 2; ++w)
        while ((int)h->ev[k][w].size() < capacity) {
          hipEvent_t e;
          if (hipEventCreate(&e) != hipSuccess) return FFN_E_HIP;
          h->ev[k][w].push_back(e);
        }
    h->cap = capacity;
  }
  for (int k = 0; k < FFN_K_COUNT; ++k) h->used[k] = 0;
  h->timing = true;
  return FFN_OK;
}

ffn_status ffn_sparse_timing_read(ffn_sparse_handle* h, int32_t kind, int32_t* launches, double* total_ms) {
  if (!h || kind < 0 || kind >= FFN_K_COUNT || !launches || !total_ms) return FFN_E_INVALID;
  double tot = 0.0;
  const int n = h->used[kind];
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(h->ev[kind][1][i]) != hipSuccess) return FFN_E_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, h->ev[kind][0][i], h->ev[kind][1][i]) != hipSuccess) return FFN_E_HIP;
    tot += ms;
  }
  *launches = n;
  *total_ms = tot;
  h->used[kind] = 0;
  return FFN_OK;
}

void ffn_sparse_destroy(ffn_sparse_handle* h) {
  if (!h) return;
  for (int k = 0; k < FFN_K_COUNT; ++k)
    for (int w = 0; w < 2; ++w)
      for (hipEvent_t e : h->ev[k][w]) (void)hipEventDestroy(e);
  delete h;
}

}  // extern "C"
