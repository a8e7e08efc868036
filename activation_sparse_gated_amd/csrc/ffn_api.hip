// C ABI of the sparse gated FFN library: argument checks, workspace layout,
// kernel planning and launches. Everything here runs on the host; every step
// of the computation runs in the kernels of k_gate / k_updown / k_topk.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/ffn_sparse.h"
#include "kernels.cuh"

using namespace ffn;

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

struct Workspace {
  uint32_t* ctrl;       // kCtrlWords control words + kTicketWords tickets
  void* wdown_alt;      // the W_down layout the caller did not pass
  float* colnorm;       // [F]
  float* lr_t;          // [max_m x rank]
  float* lr_t_fb;       // [max_m x rank] (dense backup)
  float* g_ext;         // [max_m x F] low-rank gate values of the dense paths
  float* splitk;        // split-K partial tiles
  size_t splitk_floats;
  float* wina_s;        // [max_m x F]
  float* wina_h;        // [max_m x F]
  uint64_t* lb;         // [max_m x F / 16]
  int32_t* offs;        // [max_m + 1]
  float* ud_partial;    // [(ud_grid + max_m) x d]
  void* hbuf;           // [max_m x F] dense hidden
  size_t total;
};

int ud_grid_for(int cus) { return std::max(64, cus); }

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
  const size_t Mp = (M + 63) / 64 * 64;
  w.ctrl = (uint32_t*)take((kCtrlWords + kTicketWords) * sizeof(uint32_t));
  w.wdown_alt = take(F * d * es);
  w.colnorm = (float*)take(F * sizeof(float));
  w.lr_t = (float*)take(std::max<size_t>(1, M * r) * sizeof(float));
  w.lr_t_fb = (float*)take(std::max<size_t>(1, M * r) * sizeof(float));
  w.g_ext = (float*)take(r ? M * F * sizeof(float) : 16);
  // split-K partials: worst case is a 16-row tile split 16 ways over every row
  // of the larger of rank / d_model, for all token blocks
  w.splitk_floats = std::max<size_t>(r, d) * 16 * Mp + 4096;
  w.splitk = (float*)take(w.splitk_floats * sizeof(float));
  const bool topk = c.sel == FFN_SEL_TOPK_WINA;
  w.wina_s = (float*)take(topk ? M * F * sizeof(float) : 16);
  w.wina_h = (float*)take(topk ? M * F * sizeof(float) : 16);
  w.lb = (uint64_t*)take(M * (F / 16) * sizeof(uint64_t));
  w.offs = (int32_t*)take((M + 1) * sizeof(int32_t));
  w.ud_partial = (float*)take((ud_grid_for(cus) + M) * d * sizeof(float));
  w.hbuf = take(M * F * es);
  w.total = off;
  return w;
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

struct ffn_sparse_handle {
  ffn_sparse_config cfg;
  const void *w_gate, *u, *v, *w_up, *w_down_om, *w_down_nm;
  Workspace ws;
  int cus;
  // timing
  bool timing = false;
  int cap = 0;
  std::vector<hipEvent_t> ev[FFN_K_COUNT][2];
  int used[FFN_K_COUNT] = {};
};

namespace {

struct Timed {
  ffn_sparse_handle* h;
  int kind;
  hipStream_t s;
  bool on;
  Timed(ffn_sparse_handle* hh, int k, hipStream_t st) : h(hh), kind(k), s(st) {
    on = h->timing && h->used[kind] < h->cap;
    if (on) (void)hipEventRecord(h->ev[kind][0][h->used[kind]], s);
  }
  ~Timed() {
    if (on) {
      (void)hipEventRecord(h->ev[kind][1][h->used[kind]], s);
      h->used[kind]++;
    }
  }
};

ffn_status hip_status(hipError_t e) { return e == hipSuccess ? FFN_OK : FFN_E_HIP; }

GemmDesc gemm_base(const ffn_sparse_handle* h) {
  GemmDesc g{};
  g.dtype = h->cfg.dtype;
  g.nmat = 1;
  g.ks = 1;
  g.partial = h->ws.splitk;
  g.tickets = h->ws.ctrl + kCtrlWords;
  g.ctrl = h->ws.ctrl;
  g.bmode = B_NATIVE;
  return g;
}

// Fills nt / mt / ks for a GEMM of nrows x nmat rows, K, M tokens.
bool plan(GemmDesc& g, const ffn_sparse_handle* h, int T, int want_wg) {
  const bool f32 = g.dtype == FFN_F32;
  g.mt = f32 ? 16 : pick_mt(g.M);
  const int mblocks = ceil_div(g.M, g.mt);
  g.nt = pick_nt(g.nrows, g.nmat, T, mblocks, want_wg, f32);
  if (g.nt == 0) return false;
  const int tiles = g.nrows * g.nmat / g.nt;
  g.ks = 1;
  if (!f32) {
    const int kch = g.K / 32;
    while (tiles * mblocks * g.ks < want_wg && g.ks < 16 && kch / (g.ks * 2) >= 4) g.ks *= 2;
    const size_t need = (size_t)tiles * mblocks * g.ks * g.nt * g.mt;
    if (need > h->ws.splitk_floats || (size_t)tiles * mblocks > (size_t)kTicketWords) g.ks = 1;
  }
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

// t = V x for `m` token slots (optionally gathered), fp32 out.
hipError_t run_lowrank_v(ffn_sparse_handle* h, const void* x, int m, const int32_t* gather,
                         const int32_t* m_dev, float* t_out, hipStream_t s) {
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
  if (!plan(g, h, 0, h->cus)) return hipErrorInvalidValue;
  EpiDesc e{};
  e.kind = EPI_STORE_F32;
  e.F = c.rank;
  e.out = t_out;
  e.ldo = c.rank;
  Timed tm(h, FFN_K_LOWRANK_V, s);
  return launch_gemm(g, e, s);
}

// Dense hidden h (bf16/fp32 [slots x F] in hbuf) for `m` slots; gathered when
// `list` is set (dense backup) with the device count m_dev.
hipError_t run_dense_hidden(ffn_sparse_handle* h, const void* x, int m, const int32_t* list,
                            const int32_t* m_dev, const float* bias, float bias_scalar,
                            const float* tau, int kind, hipStream_t s) {
  const auto& c = h->cfg;
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
    if (!plan(g, h, 0, h->cus)) return hipErrorInvalidValue;
    Timed tm(h, kind, s);
    return launch_gemm(g, e, s);
  }
  // low-rank gate: t = V x, g = U t (fp32 into g_ext), then the up GEMM
  float* t = list ? h->ws.lr_t_fb : h->ws.lr_t;
  hipError_t err = run_lowrank_v(h, x, m, list, m_dev, t, s);
  if (err != hipSuccess) return err;
  {
    GemmDesc gu = gemm_base(h);
    gu.A0 = h->u;
    gu.nrows = c.d_ff;
    gu.lda = c.rank;
    gu.K = c.rank;
    gu.B = t;
    gu.ldb = c.rank;
    gu.bmode = c.dtype == FFN_BF16 ? B_F32_SPLIT : B_NATIVE;
    gu.M = m;
    gu.m_dev = m_dev;
    if (!plan(gu, h, 0, h->cus)) return hipErrorInvalidValue;
    EpiDesc eg{};
    eg.kind = EPI_STORE_F32;
    eg.F = c.d_ff;
    eg.out = h->ws.g_ext;
    eg.ldo = c.d_ff;
    Timed tm(h, kind, s);
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
  if (!plan(g, h, 0, h->cus)) return hipErrorInvalidValue;
  Timed tm(h, kind, s);
  return launch_gemm(g, e, s);
}

// y rows = W_down h for `m` slots of hbuf (scattered through `list`).
hipError_t run_dense_down(ffn_sparse_handle* h, int m, const int32_t* list, const int32_t* m_dev,
                          void* y, int kind, hipStream_t s) {
  const auto& c = h->cfg;
  GemmDesc g = gemm_base(h);
  g.A0 = h->w_down_om;
  g.nrows = c.d_model;
  g.lda = c.d_ff;
  g.K = c.d_ff;
  g.B = h->ws.hbuf;
  g.ldb = c.d_ff;
  g.M = m;
  g.m_dev = m_dev;
  if (!plan(g, h, 0, h->cus)) return hipErrorInvalidValue;
  EpiDesc e{};
  e.kind = EPI_Y;
  e.F = c.d_model;
  e.out_f32 = c.dtype == FFN_F32;
  e.y = y;
  e.ldy = c.d_model;
  e.yrows = list;
  Timed tm(h, kind, s);
  return launch_gemm(g, e, s);
}

UpdownDesc updown_desc(const ffn_sparse_handle* h, const void* x, int m, const ffn_twell_pack* p, void* y) {
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
  u.route = p->route;
  u.offs = h->ws.offs;
  u.y = y;
  u.partial = h->ws.ud_partial;
  u.grid = ud_grid_for(h->cus);
  u.min_chunk = 8;
  return u;
}

}  // namespace

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
  if (c->dtype == FFN_F32 && c->tile_w % 32 != 0 && c->tile_w != 16) return FFN_E_UNSUPPORTED;
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
  ffn_sparse_handle* h = new (std::nothrow) ffn_sparse_handle();
  if (!h) return FFN_E_INVALID;
  h->cfg = *cfg;
  h->ws = ws;
  h->cus = cus;
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
  if (err == hipSuccess) err = launch_fill_u32(ws.ctrl, 0u, kCtrlWords + kTicketWords, s);
  if (err == hipSuccess)
    err = launch_fill_u32(reinterpret_cast<uint32_t*>(ws.lb), 0u,
                          (size_t)cfg->max_m * (cfg->d_ff / 16) * 2, s);
  if (err != hipSuccess) {
    delete h;
    return FFN_E_HIP;
  }
  *out = h;
  return FFN_OK;
}

ffn_status ffn_sparse_gate_pack(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                                float bias_scalar, const float* tau, int32_t k, ffn_twell_pack* pack,
                                float* g_debug, float* s_debug, void* stream) {
  ffn_status st = check_call(h, x, m, tau, k);
  if (st != FFN_OK) return st;
  if (!pack_ok(pack)) return FFN_E_INVALID;
  const auto& c = h->cfg;
  if (s_debug && c.sel != FFN_SEL_TOPK_WINA) return FFN_E_INVALID;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (m == 0) {
    hipError_t e1 = launch_fill_u32(reinterpret_cast<uint32_t*>(pack->n_dense), 0u, 1, s);
    hipError_t e2 = launch_fill_u32(reinterpret_cast<uint32_t*>(h->ws.offs), 0u, 1, s);
    return hip_status(e1 != hipSuccess ? e1 : e2);
  }
  EpiDesc e = epi_base(h, bias, bias_scalar, tau);
  e.g_debug = g_debug;
  e.s_debug = s_debug;
  e.cnt = pack->cnt;
  e.idx = pack->idx;
  e.val = pack->val;
  e.route = pack->route;
  e.dense_list = pack->dense_list;
  e.n_dense = pack->n_dense;
  e.offs = h->ws.offs;
  e.lb = h->ws.lb;
  GemmDesc g = gemm_base(h);
  g.M = m;
  hipError_t err = hipSuccess;
  if (c.sel == FFN_SEL_TOPK_WINA) {
    g.A0 = h->w_gate;
    g.A1 = h->w_up;
    g.nmat = 2;
    g.nrows = c.d_ff;
    g.lda = c.d_model;
    g.K = c.d_model;
    g.B = x;
    g.ldb = c.d_model;
    if (!plan(g, h, 0, h->cus)) return FFN_E_UNSUPPORTED;
    e.kind = EPI_WINA;
    e.colnorm = h->ws.colnorm;
    e.s_buf = h->ws.wina_s;
    e.h_buf = h->ws.wina_h;
    {
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
    td.offs = h->ws.offs;
    td.ctrl = h->ws.ctrl;
    Timed tm(h, FFN_K_TOPK, s);
    return hip_status(launch_topk(td, s));
  }
  if (c.rank > 0) {
    err = run_lowrank_v(h, x, m, nullptr, nullptr, h->ws.lr_t, s);
    if (err != hipSuccess) return FFN_E_HIP;
    g.A0 = h->u;
    g.lda = c.rank;
    g.K = c.rank;
    g.B = h->ws.lr_t;
    g.ldb = c.rank;
    g.bmode = c.dtype == FFN_BF16 ? B_F32_SPLIT : B_NATIVE;
  } else {
    g.A0 = h->w_gate;
    g.lda = c.d_model;
    g.K = c.d_model;
    g.B = x;
    g.ldb = c.d_model;
  }
  g.nrows = c.d_ff;
  if (!plan(g, h, c.tile_w, h->cus)) return FFN_E_UNSUPPORTED;
  e.kind = EPI_TWELL;
  Timed tm(h, FFN_K_GATE, s);
  return hip_status(launch_gemm(g, e, s));
}

ffn_status ffn_sparse_updown(ffn_sparse_handle* h, const void* x, int32_t m, const ffn_twell_pack* pack,
                             void* y, void* stream) {
  ffn_status st = check_call(h, x, m, reinterpret_cast<const float*>(1), 0);
  if (st != FFN_OK) return st;
  if (!pack_ok(pack) || (m > 0 && (!y || !aligned16(y)))) return FFN_E_INVALID;
  if (m == 0) return FFN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  UpdownDesc u = updown_desc(h, x, m, pack, y);
  hipError_t err;
  {
    Timed tm(h, FFN_K_UPDOWN, s);
    err = launch_updown(u, s);
  }
  if (err != hipSuccess) return FFN_E_HIP;
  Timed tm(h, FFN_K_REDUCE, s);
  return hip_status(launch_updown_reduce(u, s));
}

ffn_status ffn_sparse_dense_fallback(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
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

ffn_status ffn_sparse_forward(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
                              float bias_scalar, const float* tau, int32_t k, ffn_twell_pack* pack,
                              void* y, void* stream) {
  ffn_status st = ffn_sparse_gate_pack(h, x, m, bias, bias_scalar, tau, k, pack, nullptr, nullptr, stream);
  if (st != FFN_OK) return st;
  st = ffn_sparse_updown(h, x, m, pack, y, stream);
  if (st != FFN_OK) return st;
  return ffn_sparse_dense_fallback(h, x, m, bias, bias_scalar, tau, k, pack, y, stream);
}

ffn_status ffn_sparse_dense_forward(ffn_sparse_handle* h, const void* x, int32_t m, const float* bias,
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
