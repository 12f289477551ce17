// atlas_mem_api.hip -- host side of the C ABI declared in include/atlas_mem.h:
// configuration checks, kernel selection, workspace, state layout, launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "atlas_mem.h"
#include "atlas_mem_internal.h"
#include "atlas_mem_linear.h"

namespace atlas {

typedef hipError_t (*LaunchFn)(const ChunkParams&, const CoeffParams&, int, hipStream_t, hipEvent_t, hipEvent_t);

struct Variant {
  const char* name;
  int io, mem, phi, dk, dv, h, bc, wp, pd;
  size_t ws_bytes;
  LaunchFn launch;
};

template <typename T> constexpr int io_code() { return sizeof(T) == 4 ? ATLAS_F32 : ATLAS_BF16; }

#define ATLAS_VARIANT(NAME, T, TI, MEM, PHI, DK, DV, H, BC, WP, PD)                          \
  {#NAME, io_code<TI>(), MEM, PHI, DK, DV, H, BC, WP, PD,                                     \
   Shape<T, TI, MEM, PHI, DK, DV, H, BC, WP, PD>::WS::bytes,                                  \
   &launch<Shape<T, TI, MEM, PHI, DK, DV, H, BC, WP, PD>>},
static const Variant kVariants[] = {
#include "atlas_mem_variants.inc"
};
#undef ATLAS_VARIANT

typedef hipError_t (*ShardedLaunchFn)(const ShardedParams&, const CoeffParams&, hipStream_t, hipEvent_t, hipEvent_t);

struct ShardedVariant {
  const char* name;
  int d, dv, h, g, wp, bc;
  size_t (*xbytes)();
  ShardedLaunchFn launch;
};

#define ATLAS_SHARDED(NAME, D, DV, H, G, WP, BC) \
  {#NAME, D, DV, H, G, WP, BC, &sharded_xbytes<D, DV, H, G, WP, BC>, &launch_sharded<D, DV, H, G, WP, BC>},
static const ShardedVariant kSharded[] = {
#include "atlas_mem_sharded_variants.inc"
};
#undef ATLAS_SHARDED

struct StreamVariant {
  const char* name;
  int d, dv, h, wp, bc, g, autopick;
  size_t (*xbytes)();
  ShardedLaunchFn launch;
};

#define ATLAS_STREAMED(NAME, D, DV, H, WP, BC, G, AUTO) \
  {#NAME, D, DV, H, WP, BC, G, AUTO, &streamed_xbytes<D, DV, H, WP, BC, G>, &launch_streamed<D, DV, H, WP, BC, G>},
static const StreamVariant kStreamed[] = {
#include "atlas_mem_stream_variants.inc"
};
#undef ATLAS_STREAMED

typedef hipError_t (*GroupedLaunchFn)(const GroupedParams&, const CoeffParams&, hipStream_t, hipEvent_t, hipEvent_t);

struct GroupedVariant {
  const char* name;
  int phi, dk, pd, dv, h, g, wp;   // h = 0: linear memory
  size_t (*seq_bytes)(int);
  GroupedLaunchFn launch;
};

#define ATLAS_GROUPED(NAME, PHI, DK, PD, DV, H, G) \
  {#NAME, PHI, DK, PD, DV, H, G, 128, &grouped_seq_bytes<PHI, DK, PD, DV, H, G>, &launch_grouped<PHI, DK, PD, DV, H, G>},
#define ATLAS_LINEAR(NAME, PHI, DK, PD, DV, WP) \
  {#NAME, PHI, DK, PD, DV, 0, 1, WP, &linear_seq_bytes<PHI, DK, PD, DV, WP>, &launch_linear<PHI, DK, PD, DV, WP>},
static const GroupedVariant kGrouped[] = {
#include "atlas_mem_grouped_variants.inc"
};
#undef ATLAS_GROUPED
#undef ATLAS_LINEAR

}  // namespace atlas

using namespace atlas;

struct atlas_mem_s {
  uint32_t magic;
  atlas_mem_config cfg;
  const Variant* var;           // per-sequence kernel, or
  const ShardedVariant* svar;   // sharded kernel, or
  const StreamVariant* tvar;    // streamed-state kernel, or
  const GroupedVariant* gvar;   // grouped kernel (wide feature maps)
  unsigned* ctrl;               // sharded: error word + barrier counters
  atlas_mem_state_layout lay;
  int n_seq, nchunks, coef_stride, device;
  char* ws;
  float* coef;
  hipEvent_t ev_before, ev_after;
  char* mws;           // Muon: per-workgroup workspace inside ws (else null)
  size_t mws_stride;
  int group;           // workgroups per sequence of the per-sequence family (2: Muon on an MLP)
};

static const uint32_t kMagic = 0xA7A5AE11u;
static thread_local char g_hip_error[256] = "";

static atlas_status hip_fail(hipError_t e) {
  std::snprintf(g_hip_error, sizeof(g_hip_error), "%s", hipGetErrorString(e));
  return ATLAS_ERR_HIP;
}

namespace atlas {
// the message atlas_mem_last_hip_error returns (other translation units)
void record_hip_error(const char* what) { std::snprintf(g_hip_error, sizeof(g_hip_error), "%s", what); }
}  // namespace atlas

static int pd_of(const atlas_mem_config* c) {
  return c->feature_map == ATLAS_PHI_POLY2 ? c->d_k : c->feature_map == ATLAS_PHI_RAW_POLY2 ? c->poly_dims : 0;
}

static const ShardedVariant* find_sharded(const atlas_mem_config* c) {
  if (c->memory != ATLAS_MEM_MLP || c->feature_map != ATLAS_PHI_IDENTITY || c->io_dtype != ATLAS_BF16) return nullptr;
  if (c->bias != ATLAS_BIAS_L2 && c->bias != ATLAS_BIAS_DOT) return nullptr;
  if (c->mlp_layernorm || c->mlp_gated) return nullptr;
  if (c->d_k != c->d_v) return nullptr;
  const int need_w = c->chunk + c->window - 1;
  const ShardedVariant* best = nullptr;
  for (const ShardedVariant& v : kSharded) {
    if (v.d != c->d_k || v.dv != c->d_v || v.h != c->mlp_hidden || v.bc != c->chunk || v.wp < need_w) continue;
    if (!best || v.wp < best->wp) best = &v;
  }
  return best;
}

static const StreamVariant* find_streamed(const atlas_mem_config* c) {
  if (c->memory != ATLAS_MEM_MLP || c->feature_map != ATLAS_PHI_IDENTITY || c->io_dtype != ATLAS_BF16) return nullptr;
  if (c->mlp_gated) return nullptr;
  if (c->d_k != c->d_v) return nullptr;
  // the kernel addresses one sequence's inputs and coefficients through
  // 32-bit buffer offsets (below 1 GiB each)
  const size_t nch = ((size_t)c->seq_len + c->chunk - 1) / c->chunk;
  if ((size_t)c->seq_len * c->d_k * 2 > (1u << 30) || nch * coef_stride(c->chunk, c->chunk + c->window - 1 + 31, true, true) * 4 > (1u << 30))
    return nullptr;
  const int need_w = c->chunk + c->window - 1;
  const StreamVariant* best = nullptr;
  for (const StreamVariant& v : kStreamed) {
    if (v.d != c->d_k || v.dv != c->d_v || v.h != c->mlp_hidden || v.bc != c->chunk || v.wp < need_w) continue;
    if (!best || v.wp < best->wp) best = &v;
  }
  return best;
}

static const GroupedVariant* find_grouped(const atlas_mem_config* c) {
  if (c->io_dtype != ATLAS_BF16 || c->optimizer != ATLAS_OPT_GD) return nullptr;
  if (c->bias != ATLAS_BIAS_L2 && c->bias != ATLAS_BIAS_DOT) return nullptr;
  if (c->mlp_layernorm || c->mlp_gated) return nullptr;
  if (c->chunk != 64 || c->window > 64) return nullptr;
  const int h = c->memory == ATLAS_MEM_MLP ? c->mlp_hidden : 0;
  const int nch = (c->seq_len + c->chunk - 1) / c->chunk;
  const GroupedVariant* best = nullptr;
  for (const GroupedVariant& v : kGrouped) {
    if (v.phi != c->feature_map || v.dk != c->d_k || v.pd != pd_of(c) || v.dv != c->d_v || v.h != h) continue;
    if (v.wp < c->chunk + c->window - 1) continue;
    if (!best || v.wp < best->wp) best = &v;
  }
  // the kernels address one sequence's workspace through 32-bit offsets
  if (best && best->seq_bytes(nch) >= (1u << 31)) return nullptr;
  return best;
}

// Exactly one of *out, *sout, *tout, *gout is set on success.
static atlas_status check_config(const atlas_mem_config* c, const Variant** out, const ShardedVariant** sout,
                                 const StreamVariant** tout, const GroupedVariant** gout) {
  if (!c) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->batch < 1 || c->heads < 1 || c->seq_len < 0 || c->d_k < 1 || c->d_v < 1) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->window < 1 || c->chunk < 1) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->memory != ATLAS_MEM_LINEAR && c->memory != ATLAS_MEM_MLP) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->feature_map < ATLAS_PHI_IDENTITY || c->feature_map > ATLAS_PHI_RAW_POLY2) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->bias < ATLAS_BIAS_L2 || c->bias > ATLAS_BIAS_HUBER) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->bias == ATLAS_BIAS_LP && !(c->bias_p >= 1.f && c->bias_p < 1e6f)) return ATLAS_ERR_INVALID_ARGUMENT;
  if ((c->bias == ATLAS_BIAS_LP || c->bias == ATLAS_BIAS_HUBER) && !(c->sign_alpha >= 0.f && c->sign_alpha < 1e30f))
    return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->mlp_layernorm != 0 && c->mlp_layernorm != 1) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->mlp_layernorm && (c->memory != ATLAS_MEM_MLP || !(c->ln_eps > 0.f && c->ln_eps < 1.f)))
    return ATLAS_ERR_INVALID_ARGUMENT;
  if ((c->mlp_gated != 0 && c->mlp_gated != 1) || (c->mlp_gated && c->memory != ATLAS_MEM_MLP))
    return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->io_dtype != ATLAS_BF16 && c->io_dtype != ATLAS_F32) return ATLAS_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(c->grad_scale)) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->optimizer != ATLAS_OPT_GD && c->optimizer != ATLAS_OPT_MUON) return ATLAS_ERR_INVALID_ARGUMENT;
  const bool muon = c->optimizer == ATLAS_OPT_MUON;
  if (muon && (c->ns_steps < 1 || c->ns_steps > 64)) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->feature_map == ATLAS_PHI_RAW_POLY2 && (c->poly_dims < 1 || c->poly_dims > c->d_k)) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->memory == ATLAS_MEM_MLP) {
    if (c->mlp_hidden < 1) return ATLAS_ERR_INVALID_ARGUMENT;
    if (c->mlp_residual && c->d_k != c->d_v) return ATLAS_ERR_INVALID_ARGUMENT;
    if (c->mlp_layers != 2) return ATLAS_ERR_UNSUPPORTED;
  }
  if (c->window > c->chunk) return ATLAS_ERR_UNSUPPORTED;
  // sequences x chunks must fit one grid dimension of the coefficient kernel
  const long n_seq = (long)c->batch * c->heads;
  if (n_seq > (1L << 20) || n_seq * ((c->seq_len + c->chunk - 1) / c->chunk) > 0x7fffffffL) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->kernel < ATLAS_KERNEL_AUTO || c->kernel > ATLAS_KERNEL_GROUPED) return ATLAS_ERR_INVALID_ARGUMENT;
  if (out) *out = nullptr;
  if (sout) *sout = nullptr;
  if (tout) *tout = nullptr;
  if (gout) *gout = nullptr;
  // Muon: the per-sequence family, plain linear or MLP memory
  if (muon && (c->mlp_layernorm || c->mlp_gated || (c->kernel != ATLAS_KERNEL_AUTO && c->kernel != ATLAS_KERNEL_PER_SEQUENCE)))
    return ATLAS_ERR_UNSUPPORTED;
  const StreamVariant* tv = nullptr;
  if (!muon && (c->kernel == ATLAS_KERNEL_STREAMED || c->kernel == ATLAS_KERNEL_AUTO)) {
    tv = find_streamed(c);
    if (tv && (c->kernel == ATLAS_KERNEL_STREAMED || tv->autopick)) {
      if (tout) *tout = tv;
      return ATLAS_OK;
    }
    if (c->kernel == ATLAS_KERNEL_STREAMED) return ATLAS_ERR_UNSUPPORTED;
  }
  if (!muon && c->kernel != ATLAS_KERNEL_PER_SEQUENCE && c->kernel != ATLAS_KERNEL_GROUPED) {
    const ShardedVariant* sv = find_sharded(c);
    if (sv) {
      if (sout) *sout = sv;
      return ATLAS_OK;
    }
    if (c->kernel == ATLAS_KERNEL_SHARDED) return ATLAS_ERR_UNSUPPORTED;
  }
  // AUTO without a sharded kernel (l_p, Huber): a streamed one still beats
  // the per-sequence family
  if (c->kernel == ATLAS_KERNEL_AUTO && tv) {
    if (tout) *tout = tv;
    return ATLAS_OK;
  }
  // wide feature maps: the grouped family
  if (!muon && (c->kernel == ATLAS_KERNEL_AUTO || c->kernel == ATLAS_KERNEL_GROUPED)) {
    const GroupedVariant* gv = find_grouped(c);
    if (gv) {
      if (gout) *gout = gv;
      return ATLAS_OK;
    }
    if (c->kernel == ATLAS_KERNEL_GROUPED) return ATLAS_ERR_UNSUPPORTED;
  }
  const int h = c->memory == ATLAS_MEM_MLP ? c->mlp_hidden : 0;
  const int need_w = c->chunk + c->window - 1;
  const Variant* best = nullptr;
  for (const Variant& v : kVariants) {
    if (v.io != c->io_dtype || v.mem != c->memory || v.phi != c->feature_map || v.dk != c->d_k ||
        v.dv != c->d_v || v.h != h || v.bc != c->chunk || v.pd != pd_of(c))
      continue;
    if (v.wp < need_w) continue;
    if (!best || v.wp < best->wp) best = &v;
  }
  if (!best) return ATLAS_ERR_UNSUPPORTED;
  if (out) *out = best;
  return ATLAS_OK;
}

static atlas_mem_state_layout make_layout(const atlas_mem_config* c) {
  atlas_mem_state_layout L;
  const int pd = pd_of(c);
  L.feature_dim = feature_dim(c->feature_map, c->d_k, pd);
  const long D = L.feature_dim;
  L.param_count = c->memory == ATLAS_MEM_MLP
                      ? (long)c->mlp_hidden * D * (c->mlp_gated ? 2 : 1) + (long)c->d_v * c->mlp_hidden
                      : (long)c->d_v * D;
  const size_t P = (size_t)L.param_count, halo = (size_t)(c->window - 1);
  L.weights = 0;
  L.momentum = align_up(L.weights + P * 4, 16);
  L.halo_k = align_up(L.momentum + (c->momentum ? P * 4 : 0), 16);
  L.halo_v = align_up(L.halo_k + halo * c->d_k * 4, 16);
  L.halo_g = align_up(L.halo_v + halo * c->d_v * 4, 16);
  L.halo_d = align_up(L.halo_g + halo * 4, 16);
  L.count = align_up(L.halo_d + (c->bias == ATLAS_BIAS_HUBER ? halo * 4 : 0), 16);
  L.seq_stride = align_up(L.count + 8, 256);
  return L;
}

// Fields of a handle that depend on the configuration only.
static atlas_status setup_handle(const atlas_mem_config* cfg, atlas_mem_s* h) {
  const Variant* var = nullptr;
  const ShardedVariant* svar = nullptr;
  const StreamVariant* tvar = nullptr;
  const GroupedVariant* gvar = nullptr;
  atlas_status s = check_config(cfg, &var, &svar, &tvar, &gvar);
  if (s != ATLAS_OK) return s;
  *h = atlas_mem_s();
  h->magic = kMagic;
  h->cfg = *cfg;
  h->var = var;
  h->svar = svar;
  h->tvar = tvar;
  h->gvar = gvar;
  h->ctrl = nullptr;
  h->lay = make_layout(cfg);
  h->n_seq = cfg->batch * cfg->heads;
  h->nchunks = (cfg->seq_len + cfg->chunk - 1) / cfg->chunk;
  h->coef_stride = var ? coef_stride(var->bc, var->wp)
                 : svar ? coef_stride(svar->bc, svar->wp, true)
                 : tvar ? coef_stride(tvar->bc, tvar->wp, true, true)
                        : coef_stride(64, gvar->wp, true);
  h->device = -1;
  h->ws = nullptr;
  h->coef = nullptr;
  h->ev_before = h->ev_after = nullptr;
  h->mws = nullptr;
  const bool muon = cfg->optimizer == ATLAS_OPT_MUON;
  // Muon on the MLP memory: a pair of workgroups per sequence, each with its
  // own chunk and Muon workspaces, and the pair's counters after them
  h->group = muon && cfg->memory == ATLAS_MEM_MLP ? 2 : 1;
  h->mws_stride = muon ? muon_ws_of(cfg->memory == ATLAS_MEM_MLP, h->lay.feature_dim, cfg->d_v, cfg->mlp_hidden,
                                    cfg->chunk).bytes
                       : 0;
  return ATLAS_OK;
}

// Device memory a handle's calls use besides their arguments: the kernel
// workspace (ws_bytes, with the control words inside it at ctrl_off) and the
// coefficient blocks (coef_bytes).
struct WsPlan {
  size_t ws_bytes, coef_bytes, ctrl_off, mws_off;
  bool has_ctrl;
};

static WsPlan plan_workspace(const atlas_mem_s* h) {
  WsPlan pl;
  // sharded, and streamed: exchange buffers / state blocks per sequence, then
  // the control words (error word, one barrier counter per sequence, one XCD
  // mask per sequence)
  const bool grouped = h->svar || h->tvar || h->gvar;
  const size_t xbytes = h->svar   ? h->svar->xbytes()
                        : h->tvar ? h->tvar->xbytes()
                        : h->gvar ? h->gvar->seq_bytes(h->nchunks)
                                  : 0;
  const size_t ctrl_grouped = align_up(xbytes * (size_t)h->n_seq, 256);
  const size_t members = (size_t)h->n_seq * h->group;
  pl.mws_off = h->var ? align_up(h->var->ws_bytes * members, 256) : 0;
  const size_t pctrl_off = align_up(pl.mws_off + h->mws_stride * members, 256);
  const size_t ctrl_bytes = align_up((1 + 2 * (size_t)h->n_seq) * 4, 256);
  pl.ws_bytes = h->var ? pctrl_off + (h->group > 1 ? ctrl_bytes : 0) : grouped ? ctrl_grouped + ctrl_bytes : 0;
  pl.ctrl_off = h->var ? pctrl_off : ctrl_grouped;
  pl.has_ctrl = grouped || h->group > 1;
  pl.coef_bytes = (size_t)h->n_seq * h->nchunks * h->coef_stride * sizeof(float);
  return pl;
}

static void bind_workspace(atlas_mem_s* h, const WsPlan& pl, char* ws, float* coef) {
  h->ws = ws;
  h->coef = coef;
  h->mws = h->cfg.optimizer == ATLAS_OPT_MUON ? ws + pl.mws_off : nullptr;
  h->ctrl = pl.has_ctrl ? reinterpret_cast<unsigned*>(ws + pl.ctrl_off) : nullptr;
}

// ---- workspace of the allocation-free entry point
// One static buffer per device; host code never passes its name to a kernel:
// the address comes from hipGetSymbolAddress, once per device, with that
// device current.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static char* g_scratch_ptr[kMaxDevices] = {};

static hipError_t scratch_of(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// *dst = the call's error word, or 0 when the call has none
__global__ void copy_error_word(unsigned* dst, const unsigned* ctrl) {
  if (threadIdx.x == 0) *dst = ctrl ? ctrl[0] : 0u;
}

extern "C" {

atlas_status atlas_mem_supported(const atlas_mem_config* cfg) {
  return check_config(cfg, nullptr, nullptr, nullptr, nullptr);
}

atlas_status atlas_mem_init(const atlas_mem_config* cfg, atlas_mem_t* out) {
  if (!out) return ATLAS_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  atlas_mem_s tmp;
  atlas_status s = setup_handle(cfg, &tmp);
  if (s != ATLAS_OK) return s;
  hipError_t e = hipGetDevice(&tmp.device);
  if (e != hipSuccess) return hip_fail(e);
  const WsPlan pl = plan_workspace(&tmp);
  char* ws = nullptr;
  float* coef = nullptr;
  if (pl.ws_bytes && hipMalloc(&ws, pl.ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    return ATLAS_ERR_OUT_OF_MEMORY;
  }
  if (pl.coef_bytes && hipMalloc(&coef, pl.coef_bytes) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(ws);
    return ATLAS_ERR_OUT_OF_MEMORY;
  }
  bind_workspace(&tmp, pl, ws, coef);
  if (tmp.ctrl) {
    if ((e = hipMemset(tmp.ctrl, 0, (1 + 2 * (size_t)tmp.n_seq) * 4)) != hipSuccess) {
      (void)hipFree(ws);
      (void)hipFree(coef);
      return hip_fail(e);
    }
  }
  atlas_mem_s* h = new (std::nothrow) atlas_mem_s(tmp);
  if (!h) {
    (void)hipFree(ws);
    (void)hipFree(coef);
    return ATLAS_ERR_OUT_OF_MEMORY;
  }
  *out = h;
  return ATLAS_OK;
}

size_t atlas_mem_state_bytes(atlas_mem_t h) {
  if (!h || h->magic != kMagic) return 0;
  return h->lay.seq_stride * (size_t)h->n_seq;
}

atlas_status atlas_mem_state_layout_of(atlas_mem_t h, atlas_mem_state_layout* out) {
  if (!h || h->magic != kMagic || !out) return ATLAS_ERR_INVALID_ARGUMENT;
  *out = h->lay;
  return ATLAS_OK;
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

atlas_status atlas_mem_forward(atlas_mem_t h, const void* q, const void* k, const void* v,
                               const float* alpha, const float* eta, const float* theta,
                               const float* gamma, void* state, void* out, void* stream) {
  if (!h || h->magic != kMagic || h->cfg.bias == ATLAS_BIAS_HUBER) return ATLAS_ERR_INVALID_ARGUMENT;
  return atlas_mem_forward_ex(h, q, k, v, alpha, eta, theta, gamma, nullptr, state, out, stream);
}

// Checks the arguments of one call and enqueues its kernels on the workspace
// bound to h.
static atlas_status forward_impl(const atlas_mem_s* h, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* eta, const float* theta,
                                 const float* gamma, const float* delta, void* state, void* out, void* stream) {
  const atlas_mem_config& c = h->cfg;
  if (c.seq_len == 0) return ATLAS_OK;  // nothing to read or write; any pointer accepted
  if (!q || !k || !v || !alpha || !theta || !gamma || !state || !out) return ATLAS_ERR_INVALID_ARGUMENT;
  if (c.momentum && !eta) return ATLAS_ERR_INVALID_ARGUMENT;
  const bool huber = c.bias == ATLAS_BIAS_HUBER;
  if (huber && (!delta || (uintptr_t)delta % 4)) return ATLAS_ERR_INVALID_ARGUMENT;
  if (!huber) delta = nullptr;
  const void* p16[] = {q, k, v, state, out};
  for (const void* p : p16)
    if ((uintptr_t)p % 16) return ATLAS_ERR_INVALID_ARGUMENT;
  const void* p4[] = {alpha, eta, theta, gamma};
  for (const void* p : p4)
    if ((uintptr_t)p % 4) return ATLAS_ERR_INVALID_ARGUMENT;
  const size_t es = c.io_dtype == ATLAS_F32 ? 4 : 2, S = (size_t)h->n_seq, N = (size_t)c.seq_len;
  const size_t out_b = S * N * c.d_v * es;
  const size_t st_b = h->lay.seq_stride * (size_t)h->n_seq;
  if (overlaps(out, out_b, q, S * N * c.d_k * es) || overlaps(out, out_b, k, S * N * c.d_k * es) ||
      overlaps(out, out_b, v, S * N * c.d_v * es) || overlaps(out, out_b, state, st_b) ||
      overlaps(out, out_b, alpha, S * N * 4) || overlaps(out, out_b, theta, S * N * 4) ||
      overlaps(out, out_b, gamma, S * N * 4) || (eta && overlaps(out, out_b, eta, S * N * 4)) ||
      (delta && overlaps(out, out_b, delta, S * N * 4)) || (delta && overlaps(state, st_b, delta, S * N * 4)) ||
      overlaps(state, st_b, q, S * N * c.d_k * es) || overlaps(state, st_b, k, S * N * c.d_k * es) ||
      overlaps(state, st_b, v, S * N * c.d_v * es))
    return ATLAS_ERR_INVALID_ARGUMENT;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev != h->device) return ATLAS_ERR_INVALID_ARGUMENT;

  CoeffParams kp;
  kp.ctrl = h->ctrl;
  kp.q = q;
  kp.k = k;
  kp.off_halo_k = h->lay.halo_k;
  kp.alpha = alpha;
  kp.eta = eta;
  kp.theta = theta;
  kp.state = (const char*)state;
  kp.coef = h->coef;
  kp.N = c.seq_len;
  kp.c = c.window;
  kp.nchunks = h->nchunks;
  kp.coef_stride = h->coef_stride;
  kp.momentum = c.momentum;
  kp.seq_stride = h->lay.seq_stride;
  kp.off_count = h->lay.count;

  if (h->gvar) {
    GroupedParams gp;
    gp.q = q;
    gp.k = k;
    gp.v = v;
    gp.gamma = gamma;
    gp.state = (char*)state;
    gp.out = out;
    gp.gws = h->ws;
    gp.gseq_bytes = h->gvar->seq_bytes(h->nchunks);
    gp.ctrl = h->ctrl;
    gp.coef = h->coef;
    gp.n_seq = h->n_seq;
    gp.N = c.seq_len;
    gp.c = c.window;
    gp.nchunks = h->nchunks;
    gp.coef_stride = h->coef_stride;
    gp.seq_stride = h->lay.seq_stride;
    gp.off_weights = h->lay.weights;
    gp.off_momentum = h->lay.momentum;
    gp.off_halo_k = h->lay.halo_k;
    gp.off_halo_v = h->lay.halo_v;
    gp.off_halo_g = h->lay.halo_g;
    gp.off_count = h->lay.count;
    gp.grad_scale = c.grad_scale;
    gp.momentum = c.momentum;
    gp.bias = c.bias;
    gp.residual = c.mlp_residual;
    e = h->gvar->launch(gp, kp, (hipStream_t)stream, h->ev_before, h->ev_after);
    if (e != hipSuccess) return hip_fail(e);
    return ATLAS_OK;
  }
  if (h->svar || h->tvar) {
    ShardedParams sp;
    sp.q = q;
    sp.k = k;
    sp.v = v;
    sp.gamma = gamma;
    sp.state = (char*)state;
    sp.out = out;
    sp.xws = h->ws;
    sp.ctrl = h->ctrl;
    sp.coef = h->coef;
    sp.n_seq = h->n_seq;
    sp.N = c.seq_len;
    sp.c = c.window;
    sp.nchunks = h->nchunks;
    sp.coef_stride = h->coef_stride;
    sp.seq_stride = h->lay.seq_stride;
    sp.off_weights = h->lay.weights;
    sp.off_momentum = h->lay.momentum;
    sp.off_halo_k = h->lay.halo_k;
    sp.off_halo_v = h->lay.halo_v;
    sp.off_halo_g = h->lay.halo_g;
    sp.off_count = h->lay.count;
    sp.grad_scale = c.grad_scale;
    sp.momentum = c.momentum;
    sp.bias = c.bias;
    sp.bias_p = c.bias_p;
    sp.sign_alpha = c.sign_alpha;
    sp.layernorm = c.mlp_layernorm;
    sp.ln_eps = c.ln_eps;
    sp.delta = delta;
    sp.off_halo_d = h->lay.halo_d;
    sp.residual = c.mlp_residual;
    e = (h->svar ? h->svar->launch : h->tvar->launch)(sp, kp, (hipStream_t)stream, h->ev_before, h->ev_after);
    if (e != hipSuccess) return hip_fail(e);
    return ATLAS_OK;
  }
  ChunkParams cp;
  cp.q = q;
  cp.k = k;
  cp.v = v;
  cp.gamma = gamma;
  cp.state = (char*)state;
  cp.out = out;
  cp.ws = h->ws;
  cp.coef = h->coef;
  cp.N = c.seq_len;
  cp.c = c.window;
  cp.nchunks = h->nchunks;
  cp.coef_stride = h->coef_stride;
  cp.seq_stride = h->lay.seq_stride;
  cp.off_weights = h->lay.weights;
  cp.off_momentum = h->lay.momentum;
  cp.off_halo_k = h->lay.halo_k;
  cp.off_halo_v = h->lay.halo_v;
  cp.off_halo_g = h->lay.halo_g;
  cp.off_count = h->lay.count;
  cp.grad_scale = c.grad_scale;
  cp.momentum = c.momentum;
  cp.bias = c.bias;
  cp.bias_p = c.bias_p;
  cp.sign_alpha = c.sign_alpha;
  cp.layernorm = c.memory == ATLAS_MEM_MLP ? c.mlp_layernorm : 0;
  cp.gated = c.memory == ATLAS_MEM_MLP ? c.mlp_gated : 0;
  cp.ln_eps = c.ln_eps;
  cp.delta = delta;
  cp.off_halo_d = h->lay.halo_d;
  cp.residual = c.memory == ATLAS_MEM_MLP ? c.mlp_residual : 0;
  cp.alpha = alpha;
  cp.eta = c.momentum ? eta : nullptr;
  cp.theta = theta;
  cp.muon = c.optimizer == ATLAS_OPT_MUON;
  cp.ns_steps = c.ns_steps;
  cp.mws = h->mws;
  cp.mws_stride = h->mws_stride;
  cp.ctrl = h->ctrl;
  cp.n_seq = h->n_seq;
  cp.group = h->group;
  e = h->var->launch(cp, kp, h->n_seq, (hipStream_t)stream, h->ev_before, h->ev_after);
  if (e != hipSuccess) return hip_fail(e);
  return ATLAS_OK;
}

atlas_status atlas_mem_forward_ex(atlas_mem_t h, const void* q, const void* k, const void* v,
                                  const float* alpha, const float* eta, const float* theta,
                                  const float* gamma, const float* delta, void* state, void* out, void* stream) {
  if (!h || h->magic != kMagic) return ATLAS_ERR_INVALID_ARGUMENT;
  return forward_impl(h, q, k, v, alpha, eta, theta, gamma, delta, state, out, stream);
}

atlas_status atlas_mem_forward_noalloc(const atlas_mem_config* cfg, const void* q, const void* k, const void* v,
                                       const float* alpha, const float* eta, const float* theta,
                                       const float* gamma, const float* delta, void* state, void* out,
                                       unsigned* errors, void* stream) {
  atlas_mem_s h;
  atlas_status s = setup_handle(cfg, &h);
  if (s != ATLAS_OK) return s;
  if (cfg->seq_len == 0) return ATLAS_OK;
  if (errors && (uintptr_t)errors % 4) return ATLAS_ERR_INVALID_ARGUMENT;
  hipError_t e = hipGetDevice(&h.device);
  if (e != hipSuccess) return hip_fail(e);
  const WsPlan pl = plan_workspace(&h);
  const size_t coef_off = align_up(pl.ws_bytes, 256);
  if (coef_off + pl.coef_bytes > kScratchBytes) return ATLAS_ERR_SCRATCH_TOO_SMALL;
  char* base = nullptr;
  if ((e = scratch_of(h.device, &base)) != hipSuccess) return hip_fail(e);
  bind_workspace(&h, pl, base, reinterpret_cast<float*>(base + coef_off));
  // the coefficient kernel clears the control words at the start of the call
  s = forward_impl(&h, q, k, v, alpha, eta, theta, gamma, delta, state, out, stream);
  if (s != ATLAS_OK || !errors) return s;
  hipLaunchKernelGGL(copy_error_word, dim3(1), dim3(64), 0, (hipStream_t)stream, errors, (const unsigned*)h.ctrl);
  e = hipGetLastError();
  return e == hipSuccess ? ATLAS_OK : hip_fail(e);
}

atlas_status atlas_mem_set_kernel_events(atlas_mem_t h, void* before, void* after) {
  if (!h || h->magic != kMagic) return ATLAS_ERR_INVALID_ARGUMENT;
  if ((before == nullptr) != (after == nullptr)) return ATLAS_ERR_INVALID_ARGUMENT;
  h->ev_before = (hipEvent_t)before;
  h->ev_after = (hipEvent_t)after;
  return ATLAS_OK;
}

int atlas_mem_kernel_family(atlas_mem_t h) {
  if (!h || h->magic != kMagic) return -1;
  return h->var ? ATLAS_KERNEL_PER_SEQUENCE : h->svar ? ATLAS_KERNEL_SHARDED : h->tvar ? ATLAS_KERNEL_STREAMED
                                                                                    : ATLAS_KERNEL_GROUPED;
}

atlas_status atlas_mem_device_errors(atlas_mem_t h, unsigned* flags) {
  if (!h || h->magic != kMagic || !flags) return ATLAS_ERR_INVALID_ARGUMENT;
  *flags = 0;
  if (!h->ctrl) return ATLAS_OK;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(flags, h->ctrl, sizeof(unsigned), hipMemcpyDeviceToHost);
  return e == hipSuccess ? ATLAS_OK : hip_fail(e);
}

atlas_status atlas_mem_free(atlas_mem_t h) {
  if (!h) return ATLAS_OK;
  if (h->magic != kMagic) return ATLAS_ERR_INVALID_ARGUMENT;
  h->magic = 0;
  hipError_t e1 = h->ws ? hipFree(h->ws) : hipSuccess;
  hipError_t e2 = h->coef ? hipFree(h->coef) : hipSuccess;
  delete h;
  if (e1 != hipSuccess) return hip_fail(e1);
  if (e2 != hipSuccess) return hip_fail(e2);
  return ATLAS_OK;
}

const char* atlas_mem_error_string(int code) {
  switch (code) {
    case ATLAS_OK: return "success";
    case ATLAS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ATLAS_ERR_UNSUPPORTED: return "no kernel built for this configuration";
    case ATLAS_ERR_OUT_OF_MEMORY: return "out of device memory";
    case ATLAS_ERR_HIP: return "HIP runtime error";
    case ATLAS_ERR_SCRATCH_TOO_SMALL: return "the call needs more workspace than the static scratch buffer holds";
    default: return "unknown status";
  }
}

const char* atlas_mem_last_hip_error(void) { return g_hip_error; }

}  // extern "C"
