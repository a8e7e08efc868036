// C ABI of the gated subspace (GSI) linear map (include/ffn_gsi.h): argument
// checks, workspace layout, set-up launches and the per-group kernel sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "../../include/ffn_gsi.h"
#include "gsi.cuh"

using namespace ffn;

struct ffn_gsi_handle {
  ffn_gsi_config cfg;
  const uint16_t *w, *vk;
  uint16_t *vt, *img;
  float *g, *part;
  int32_t* counter;
  GsiDesc plan;
  int cus;
  bool failed = false;
  bool timing = false;
  int cap = 0;
  std::vector<hipEvent_t> ev[FFN_GSI_K_COUNT][2];
  int used[FFN_GSI_K_COUNT] = {};
};

namespace {

struct Layout {
  size_t vt, img, g, part, counter, total;
};

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

bool cfg_ok(const ffn_gsi_config* c) {
  return c && c->d_in >= 8 && c->d_in % 8 == 0 && c->d_in <= 16384 && c->d_out >= 1 && c->d_out <= (1 << 22) &&
         c->k >= 8 && c->k % 8 == 0 && c->k <= 512 && c->k <= c->d_in && c->max_m >= 1;
}

Layout layout(const ffn_gsi_config* c) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += al256(bytes);
    return at;
  };
  L.vt = take((size_t)c->k * c->d_in * 2);
  L.img = take((size_t)c->d_out * c->k * 2);
  L.g = take((size_t)kGsiMaxM * c->k * 4);
  L.part = take((size_t)2 * kGsiMaxM * gsi_max_parts(c->d_in, c->k) * 4);
  L.counter = take(4);
  L.total = o;
  return L;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The next kernel launched records this kind's event pair (timing enabled).
struct GsiTimed {
  ffn_gsi_handle* h;
  int kind;
  bool on;
  GsiTimed(ffn_gsi_handle* hh, int k) : h(hh), kind(k) {
    on = h->timing && h->used[kind] < h->cap;
    if (on) tl_launch_events = LaunchEvents{h->ev[kind][0][h->used[kind]], h->ev[kind][1][h->used[kind]]};
  }
  ~GsiTimed() {
    if (!on) return;
    if (tl_launch_events.start == nullptr) h->used[kind]++;
    else tl_launch_events = LaunchEvents{nullptr, nullptr};
  }
};

ffn_status fail(ffn_gsi_handle* h) {
  h->failed = true;
  return FFN_E_HIP;
}

}  // namespace

extern "C" {

ffn_status ffn_gsi_check_config(const ffn_gsi_config* cfg) { return cfg_ok(cfg) ? FFN_OK : FFN_E_INVALID; }

size_t ffn_gsi_workspace_bytes(const ffn_gsi_config* cfg) { return cfg_ok(cfg) ? layout(cfg).total : 0; }

ffn_status ffn_gsi_init(const ffn_gsi_config* cfg, const void* w, const void* vk, void* workspace,
                        size_t workspace_bytes, void* stream, ffn_gsi_handle** out) {
  if (!out) return FFN_E_INVALID;
  *out = nullptr;
  if (!cfg_ok(cfg) || !w || !vk || !workspace || !al16(w) || !al16(vk) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return FFN_E_INVALID;
  const Layout L = layout(cfg);
  if (workspace_bytes < L.total) return FFN_E_WORKSPACE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return FFN_E_HIP;
  ffn_gsi_handle* h = new (std::nothrow) ffn_gsi_handle();
  if (!h) return FFN_E_HIP;
  char* base = static_cast<char*>(workspace);
  h->cfg = *cfg;
  h->w = static_cast<const uint16_t*>(w);
  h->vk = static_cast<const uint16_t*>(vk);
  h->vt = reinterpret_cast<uint16_t*>(base + L.vt);
  h->img = reinterpret_cast<uint16_t*>(base + L.img);
  h->g = reinterpret_cast<float*>(base + L.g);
  h->part = reinterpret_cast<float*>(base + L.part);
  h->counter = reinterpret_cast<int32_t*>(base + L.counter);
  h->cus = cus;
  GsiDesc& p = h->plan;
  p = GsiDesc{};
  p.d = cfg->d_in;
  p.dout = cfg->d_out;
  p.k = cfg->k;
  p.w = h->w;
  p.vk = h->vk;
  p.vt = h->vt;
  p.img = h->img;
  p.g = h->g;
  p.part = h->part;
  p.counter = h->counter;
  if (!gsi_plan(p, cus) || p.nres > gsi_max_parts(cfg->d_in, cfg->k)) {
    delete h;
    return FFN_E_UNSUPPORTED;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_transpose(vk, h->vt, cfg->d_in, cfg->k, 2, s);
  if (e == hipSuccess) e = launch_gsi_image(h->w, h->vt, h->img, cfg->d_out, cfg->d_in, cfg->k, s);
  if (e == hipSuccess) e = launch_fill_u32(reinterpret_cast<uint32_t*>(h->counter), 0u, 1, s);
  if (e != hipSuccess) {
    delete h;
    return FFN_E_HIP;
  }
  *out = h;
  return FFN_OK;
}

ffn_status ffn_gsi_forward(ffn_gsi_handle* h, const void* x, int32_t m, float eps, void* y, float* rho,
                           int32_t* slow_list, int32_t* n_slow, void* stream) {
  if (!h) return FFN_E_INVALID;
  if (h->failed) return FFN_E_HIP;
  if (m < 0 || m > h->cfg.max_m || std::isnan(eps)) return FFN_E_INVALID;
  if ((rho && !al16(rho)) || (slow_list && !al16(slow_list)) || (n_slow && !al16(n_slow))) return FFN_E_INVALID;
  if (m > 0 && (!x || !y || !al16(x) || !al16(y))) return FFN_E_INVALID;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (m == 0) {
    if (n_slow && launch_fill_u32(reinterpret_cast<uint32_t*>(n_slow), 0u, 1, s) != hipSuccess) return fail(h);
    return FFN_OK;
  }
  const auto& c = h->cfg;
  for (int t0 = 0; t0 < m; t0 += kGsiMaxM) {
    GsiDesc d = h->plan;
    d.M = std::min(kGsiMaxM, m - t0);
    d.x = static_cast<const uint16_t*>(x) + (size_t)t0 * c.d_in;
    d.y = static_cast<uint16_t*>(y) + (size_t)t0 * c.d_out;
    d.eps = eps;
    d.force_slow = 0;
    d.tok0 = t0;
    d.rho = rho;
    d.slow_list = slow_list;
    d.n_slow = n_slow;
    hipError_t e;
    {
      GsiTimed tm(h, FFN_GSI_K_PROJ);
      e = launch_gsi_proj(d, s);
    }
    if (e != hipSuccess) return fail(h);
    {
      GsiTimed tm(h, FFN_GSI_K_RESID);
      e = launch_gsi_resid(d, s);
    }
    if (e != hipSuccess) return fail(h);
    {
      GsiTimed tm(h, FFN_GSI_K_OUT);
      e = launch_gsi_out(d, s);
    }
    if (e != hipSuccess) return fail(h);
  }
  return FFN_OK;
}

ffn_status ffn_gsi_dense_forward(ffn_gsi_handle* h, const void* x, int32_t m, void* y, void* stream) {
  if (!h) return FFN_E_INVALID;
  if (h->failed) return FFN_E_HIP;
  if (m < 0 || m > h->cfg.max_m) return FFN_E_INVALID;
  if (m == 0) return FFN_OK;
  if (!x || !y || !al16(x) || !al16(y)) return FFN_E_INVALID;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto& c = h->cfg;
  if (m == 1) {
    // one token: the plain weight stream of the dense products
    Sgemv1Desc d{};
    d.N = c.d_out;
    d.K = c.d_in;
    d.A = h->w;
    d.vec = static_cast<const uint16_t*>(x);
    d.epi = SG_Y;
    d.y = y;
    d.y_f32 = 0;
    if (sgemv1_plan(d, h->cus)) {
      GsiTimed tm(h, FFN_GSI_K_DENSE);
      return launch_sgemv1(d, s) == hipSuccess ? FFN_OK : fail(h);
    }
  }
  if (c.d_in % 32 == 0) {
    // several tokens: the library's dense GEMM kernels (VALU GEMV up to 8
    // tokens, matrix-core tiles beyond)
    GsiTimed tm(h, FFN_GSI_K_DENSE);
    return dense_rows_bf16(h->w, c.d_out, c.d_in, x, m, y, c.d_out, h->cus, s) == hipSuccess ? FFN_OK : fail(h);
  }
  for (int t0 = 0; t0 < m; t0 += kGsiMaxM) {
    GsiDesc d = h->plan;
    d.M = std::min(kGsiMaxM, m - t0);
    d.x = static_cast<const uint16_t*>(x) + (size_t)t0 * c.d_in;
    d.y = static_cast<uint16_t*>(y) + (size_t)t0 * c.d_out;
    d.force_slow = 1;
    GsiTimed tm(h, FFN_GSI_K_DENSE);
    if (launch_gsi_out(d, s) != hipSuccess) return fail(h);
  }
  return FFN_OK;
}

const void* ffn_gsi_image(const ffn_gsi_handle* h) { return h ? h->img : nullptr; }

ffn_status ffn_gsi_timing_enable(ffn_gsi_handle* h, int32_t enable, int32_t capacity) {
  if (!h || capacity < 0) return FFN_E_INVALID;
  if (!enable) {
    h->timing = false;
    return FFN_OK;
  }
  if (capacity > h->cap) {
    for (int k = 0; k < FFN_GSI_K_COUNT; ++k)
      for (int w = 0; w < 2; ++w)
        while ((int)h->ev[k][w].size() < capacity) {
          hipEvent_t e;
          if (hipEventCreate(&e) != hipSuccess) return FFN_E_HIP;
          h->ev[k][w].push_back(e);
        }
    h->cap = capacity;
  }
  for (int k = 0; k < FFN_GSI_K_COUNT; ++k) h->used[k] = 0;
  h->timing = true;
  return FFN_OK;
}

ffn_status ffn_gsi_timing_read(ffn_gsi_handle* h, int32_t kind, int32_t* launches, double* total_ms) {
  if (!h || kind < 0 || kind >= FFN_GSI_K_COUNT || !launches || !total_ms) return FFN_E_INVALID;
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

void ffn_gsi_destroy(ffn_gsi_handle* h) {
  if (!h) return;
  for (int k = 0; k < FFN_GSI_K_COUNT; ++k)
    for (int w = 0; w < 2; ++w)
      for (hipEvent_t e : h->ev[k][w]) (void)hipEventDestroy(e);
  delete h;
}

}  // extern "C"
