// prism_api.hip -- host side of libprism.so: configuration checks, workspace layout and
// the launch sequence of each entry point declared in include/prism.h.
#include <math.h>
#include <string.h>

#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "prism_internal.h"

namespace prism {

// ---------------------------------------------------------------------------- tracing
namespace {
struct TraceRecord {
  int stage;
  hipEvent_t start, end;
};
std::mutex g_trace_mu;
bool g_trace_on = false;
std::vector<TraceRecord> g_records;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drop_records() {
  for (auto &r : g_records) {
    hipEventSynchronize(r.end);
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.end);
  }
  g_records.clear();
}
}  // namespace

TraceScope::TraceScope(int st, hipStream_t s) : stage(st), stream(s), start(nullptr) {
  std::lock_guard<std::mutex> lk(g_trace_mu);
  if (!g_trace_on) return;
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, s) == hipSuccess) start = e;
}

TraceScope::~TraceScope() {
  if (!start) return;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, stream) == hipSuccess)
    g_records.push_back(TraceRecord{stage, (hipEvent_t)start, e});
  else
    g_event_pool.push_back((hipEvent_t)start);
}

// ---------------------------------------------------------------------------- call order
// The backward reads the O and lse that the forward left in the workspace, and both passes
// read the plan.  The library records, per workspace address, the configuration of the
// last plan and whether a forward has run on it since; a forward on a workspace with no
// plan of the same configuration, or a backward with no forward since the last plan, is
// refused before any launch.
namespace {
struct WsState {
  prism_config cfg;
  unsigned long long plan_gen, fwd_gen;  // fwd_gen == plan_gen: forward ran on this plan
};
std::mutex g_ws_mu;
std::unordered_map<uintptr_t, WsState> g_ws;
unsigned long long g_gen = 0;

// Field by field: the struct has padding (before eps) whose bytes a caller need not set.
// Floating fields compare by value (check_config has refused non-finite ones).
bool same_config(const prism_config &a, const prism_config &b) {
  return a.T == b.T && a.H == b.H && a.W == b.W && a.num_heads == b.num_heads &&
         a.head_dim == b.head_dim && a.dtype == b.dtype && a.min_edge_log2 == b.min_edge_log2 &&
         a.top_k == b.top_k && a.top_p == b.top_p && a.tau128 == b.tau128 &&
         a.tau256 == b.tau256 && a.eps == b.eps && a.score_scale == b.score_scale &&
         a.softmax_scale == b.softmax_scale && a.top_k_frac == b.top_k_frac &&
         a.fixed_shape == b.fixed_shape && a.map_exponent == b.map_exponent &&
         a.density_mode == b.density_mode && a.max_pairs == b.max_pairs;
}
}  // namespace

// ---------------------------------------------------------------------------- static scratch
// The workspace of prism_forward_static: a device array of fixed size that the library
// owns, for callers that cannot allocate.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a kernel or a copy
// (on the host it is only a stand-in for the symbol): the device address of this GPU's
// copy comes from hipGetSymbolAddress, taken once per device on its first call.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
namespace {
std::mutex g_scratch_mu;
std::unordered_map<int, void *> g_scratch_ptr;  // device -> address of its scratch copy
}  // namespace

static thread_local std::string g_last_error;

static prism_status fail(prism_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

prism_status check_config(const prism_config *cfg, Dims *d, const char **why) {
  *why = "";
  if (!cfg) {
    *why = "null configuration";
    return PRISM_ERR_ARG;
  }
  if (cfg->T <= 0 || cfg->H <= 0 || cfg->W <= 0 || cfg->num_heads <= 0 || cfg->head_dim <= 0) {
    *why = "grid sizes, heads and head_dim must be positive";
    return PRISM_ERR_ARG;
  }
  if (cfg->T % kZone || cfg->H % kZone || cfg->W % kZone) {
    *why = "T, H and W must be multiples of the 8-token zone edge";
    return PRISM_ERR_UNSUPPORTED;
  }
  if (cfg->dtype != PRISM_F32 && cfg->dtype != PRISM_BF16) {
    *why = "dtype must be PRISM_F32 or PRISM_BF16";
    return PRISM_ERR_UNSUPPORTED;
  }
  if (cfg->head_dim != 64 && cfg->head_dim != 128) {
    *why = "head_dim must be 64 or 128";
    return PRISM_ERR_UNSUPPORTED;
  }
  if (cfg->min_edge_log2 != 0 && cfg->min_edge_log2 != 1) {
    *why = "min_edge_log2 must be 0 or 1";
    return PRISM_ERR_ARG;
  }
  if (cfg->top_k < 0 || !(cfg->top_p >= 0.f) || !isfinite(cfg->top_p) ||
      !isfinite(cfg->tau128) || !isfinite(cfg->tau256) || !(cfg->eps >= 0.0) ||
      !isfinite(cfg->eps) || !isfinite(cfg->score_scale) || !isfinite(cfg->softmax_scale)) {
    *why = "top_k, top_p, tau, eps and scales must be finite and non-negative";
    return PRISM_ERR_ARG;
  }
  if (!(cfg->top_k_frac >= 0.f && cfg->top_k_frac <= 1.f) || !isfinite(cfg->map_exponent) ||
      cfg->density_mode < 0 || cfg->density_mode > 3) {
    *why = "top_k_frac must be in [0, 1], map_exponent finite, density_mode 0..3";
    return PRISM_ERR_ARG;
  }
  if (cfg->fixed_shape < 0) {
    *why = "fixed_shape must be 0 (shapes from the guidance) or a packed shape";
    return PRISM_ERR_ARG;
  }
  if (cfg->fixed_shape > 0) {
    const int f = cfg->fixed_shape, a = (f >> 4) & 3, b = (f >> 2) & 3, c = f & 3;
    if (f > 63 || a < cfg->min_edge_log2 || b < cfg->min_edge_log2 ||
        c < cfg->min_edge_log2 || a + b + c < 6 || a + b + c > 8) {
      *why = "fixed_shape must pack log2 edges >= min_edge_log2 with volume 64, 128 or 256";
      return PRISM_ERR_ARG;
    }
  }
  if (cfg->max_pairs < 0) {
    *why = "max_pairs must be 0 (Nb_max^2) or a positive pair count";
    return PRISM_ERR_ARG;
  }
  if (cfg->num_heads > 4096) {
    *why = "too many heads in one call";
    return PRISM_ERR_UNSUPPORTED;
  }
  // T * H first: each factor is below 2^31, so neither product overflows
  const long long TH = (long long)cfg->T * cfg->H;
  const long long N = TH > (long long)kMaxUnits * kUnit ? 0 : TH * cfg->W;
  if (N == 0 || N / kUnit > kMaxUnits) {
    *why = "more than 65535 64-token units per head";
    return PRISM_ERR_UNSUPPORTED;
  }
  d->T = cfg->T;
  d->H = cfg->H;
  d->W = cfg->W;
  d->heads = cfg->num_heads;
  d->D = cfg->head_dim;
  d->dtype = cfg->dtype;
  d->Dp = cfg->dtype == PRISM_BF16 ? 128 : cfg->head_dim;
  d->N = (int)N;
  d->Z = (int)(N / kZoneTok);
  d->U = (int)(N / kUnit);
  d->nb_max = d->U;
  d->nzt = cfg->T / kZone;
  d->nzh = cfg->H / kZone;
  d->nzw = cfg->W / kZone;
  d->words = (d->nb_max + 31) / 32;
  {
    const long long full = (long long)d->nb_max * d->nb_max;
    d->cap = cfg->max_pairs > 0 && cfg->max_pairs < full ? cfg->max_pairs : full;
  }
  d->elt = cfg->dtype == PRISM_BF16 ? 2 : 4;
  d->tok_stride = (size_t)cfg->num_heads * cfg->head_dim;
  d->head_stride = (size_t)cfg->head_dim;
  return PRISM_OK;
}

Layout make_layout(const Dims &d) {
  Layout L;
  memset(&L, 0, sizeof(L));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return at;
  };
  const size_t H = d.heads, N = d.N, Z = d.Z, U = d.U, NB = d.nb_max, D = d.D;
  L.pub.zone_stats = take(H * Z * 4 * sizeof(double));
  L.pub.audio_stats = take(Z * 4 * sizeof(double));
  L.pub.zone_diag = take(H * Z * 4 * sizeof(double));
  L.pub.zone_shape = take(H * Z * sizeof(int));
  L.pub.zone_block = take(H * (Z + 1) * sizeof(int));
  L.pub.block_start = take(H * NB * sizeof(int));
  L.pub.block_size = take(H * NB * sizeof(int));
  L.pub.unit_block = take(H * U * sizeof(int));
  L.pub.perm = take(H * N * sizeof(int));
  L.pub.inv_perm = take(H * N * sizeof(int));
  L.pub.qbar = take(H * NB * D * sizeof(float));
  L.pub.kbar = take(H * NB * D * sizeof(float));
  const size_t CAP = (size_t)d.cap;
  L.pub.sel_count = take(H * NB * sizeof(int));
  L.pub.csr_ptr = take(H * (NB + 1) * sizeof(int));
  L.pub.csr_col = take(H * CAP * sizeof(int));
  L.pub.csc_count = take(H * NB * sizeof(int));
  L.pub.csc_ptr = take(H * (NB + 1) * sizeof(int));
  L.pub.csc_row = take(H * CAP * sizeof(int));
  L.pub.scores = take(NB * NB * sizeof(float));
  L.pub.flags = take(H * sizeof(uint32_t));
  L.vmax = take(H * sizeof(float));
  L.sel_bits = take(H * NB * d.words * sizeof(uint32_t));
  L.csc_bits = take(H * NB * d.words * sizeof(uint32_t));
  L.tiles = take(H * U * sizeof(int2));
  L.btiles = take(H * 2 * Z * sizeof(int2));
  L.qt_count = take(H * 2 * Z * sizeof(int));
  L.qt_ptr = take(H * (2 * Z + 1) * sizeof(int));
  L.qt_list = take(H * CAP * sizeof(int));
  L.counters = take(16 * sizeof(int));
  L.delta = take(H * N * sizeof(float));
  L.lsep = take(H * N * sizeof(float));
  L.lse2 = take(H * N * sizeof(float));
  // the large per-token arrays start on 2 MiB boundaries: their placement relative to the
  // memory channels then does not depend on the sizes of the arrays before them
  auto take_big = [&](size_t bytes) {
    off = (off + ((size_t)1 << 21) - 1) & ~(((size_t)1 << 21) - 1);
    return take(bytes);
  };
  L.o32p = take_big(H * N * (size_t)d.Dp * sizeof(float));
  const size_t tensor = H * N * (size_t)d.Dp * d.elt;
  L.qp = take_big(tensor);
  L.kp = take_big(tensor);
  L.vp = take_big(tensor);
  L.dop = take_big(tensor);
  L.total = off;
  L.pub.total = off;
  L.pub.N = d.N;
  L.pub.Z = d.Z;
  L.pub.nb_max = d.nb_max;
  L.pub.pair_cap = d.cap;
  return L;
}

Scales scales_of(const prism_config *cfg, const Dims &d) {
  Scales s;
  const float inv = 1.0f / sqrtf((float)d.D);
  s.score = cfg->score_scale > 0 ? cfg->score_scale : inv;
  s.softmax = cfg->softmax_scale > 0 ? cfg->softmax_scale : inv;
  return s;
}

int resident_grid(const void *kernel, int block, int work_items) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    cus = 256;
    per_cu = 1;
  }
  const long long g = (long long)cus * per_cu;
  return (int)(g < work_items ? g : (work_items > 0 ? work_items : 1));
}

static prism_status launched(hipError_t e, const char *stage) {
  if (e != hipSuccess)
    return fail(PRISM_ERR_HIP, std::string(stage) + ": " + hipGetErrorString(e));
  return PRISM_OK;
}

}  // namespace prism

using namespace prism;

extern "C" {

size_t prism_workspace_bytes(const prism_config *cfg) {
  Dims d;
  const char *why;
  if (check_config(cfg, &d, &why) != PRISM_OK) return 0;
  return make_layout(d).total;
}

prism_status prism_plan_layout(const prism_config *cfg, prism_layout *out) {
  Dims d;
  const char *why;
  prism_status st = check_config(cfg, &d, &why);
  if (st != PRISM_OK) return fail(st, why);
  if (!out) return fail(PRISM_ERR_ARG, "null layout pointer");
  *out = make_layout(d).pub;
  return PRISM_OK;
}

prism_status prism_plan_view(const prism_config *cfg, const void *workspace,
                             prism_layout *out) {
  if (!workspace) return fail(PRISM_ERR_ARG, "null workspace");
  return prism_plan_layout(cfg, out);
}

prism_status prism_plan(const prism_config *cfg, const void *q, const void *k, const void *v,
                        int64_t tok_stride, int64_t head_stride, const float *a2v_norm,
                        void *workspace, size_t workspace_bytes, void *stream) {
  Dims d;
  const char *why;
  prism_status st = check_config(cfg, &d, &why);
  if (st != PRISM_OK) return fail(st, why);
  if (!q || !k || !v || !workspace) return fail(PRISM_ERR_ARG, "null tensor or workspace");
  if ((uintptr_t)workspace % 256) return fail(PRISM_ERR_ARG, "workspace not 256-byte aligned");
  if (tok_stride < 0 || head_stride < 0)
    return fail(PRISM_ERR_ARG, "strides must be non-negative (0 selects the dense layout)");
  if (tok_stride) d.tok_stride = (size_t)tok_stride;
  if (head_stride) d.head_stride = (size_t)head_stride;
  // the gather reads 16-byte pieces of every row
  if ((d.tok_stride * d.elt) % 16 || (d.head_stride * d.elt) % 16 ||
      ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) % 16)
    return fail(PRISM_ERR_ARG, "q, k, v must be 16-byte aligned and their strides multiples "
                               "of 16 bytes");
  Layout L = make_layout(d);
  if (workspace_bytes < L.total) return fail(PRISM_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  {
    // the launches below overwrite the previous plan: until they have all been issued the
    // workspace holds no valid plan (a failed launch leaves it without one)
    std::lock_guard<std::mutex> lk(g_ws_mu);
    g_ws.erase((uintptr_t)workspace);
  }
  Scales sc = scales_of(cfg, d);
  double *zstat = (double *)(ws + L.pub.zone_stats);
  double *astat = (double *)(ws + L.pub.audio_stats);
  if (a2v_norm) {
    if ((st = launched(launch_audio_stats(d, a2v_norm, astat, s), "audio stats"))) return st;
  }
  if ((st = launched(launch_zone_stats(d, v, cfg->density_mode, zstat, s), "zone stats")))
    return st;
  if ((st = launched(launch_quantize(d, cfg, zstat, astat, a2v_norm != nullptr, ws, L, s),
                     "quantiser")))
    return st;
  if ((st = launched(launch_gather(d, q, k, v, ws, L, s), "gather"))) return st;
  if ((st = launched(launch_tiles(d, ws, L, s), "tiles"))) return st;
  if ((st = launched(launch_scores_select(d, cfg, sc.score, ws, L, s), "selection"))) return st;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  WsState &w = g_ws[(uintptr_t)workspace];
  memcpy(&w.cfg, cfg, sizeof(prism_config));
  w.plan_gen = ++g_gen;
  w.fwd_gen = 0;
  return PRISM_OK;
}

prism_status prism_attn_fwd(const prism_config *cfg, void *workspace, size_t workspace_bytes,
                            void *o, float *lse, void *stream) {
  Dims d;
  const char *why;
  prism_status st = check_config(cfg, &d, &why);
  if (st != PRISM_OK) return fail(st, why);
  if (!o || !lse || !workspace) return fail(PRISM_ERR_ARG, "null output or workspace");
  if ((uintptr_t)workspace % 256 || (uintptr_t)o % 16 || (uintptr_t)lse % 4)
    return fail(PRISM_ERR_ARG, "workspace must be 256-byte, o 16-byte, lse 4-byte aligned");
  Layout L = make_layout(d);
  if (workspace_bytes < L.total) return fail(PRISM_ERR_WORKSPACE, "workspace too small");
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = g_ws.find((uintptr_t)workspace);
  if (it == g_ws.end() || !same_config(it->second.cfg, *cfg))
    return fail(PRISM_ERR_STATE, "prism_attn_fwd: no prism_plan of this configuration on "
                                 "this workspace");
  Scales sc = scales_of(cfg, d);
  st = launched(launch_attn_fwd(d, sc.softmax, (uint8_t *)workspace, L, o, lse,
                                (hipStream_t)stream),
                "attention forward");
  if (st == PRISM_OK) it->second.fwd_gen = it->second.plan_gen;
  return st;
}

prism_status prism_attn_bwd(const prism_config *cfg, void *workspace, size_t workspace_bytes,
                            const void *dout, void *dq, void *dk, void *dv, void *stream) {
  Dims d;
  const char *why;
  prism_status st = check_config(cfg, &d, &why);
  if (st != PRISM_OK) return fail(st, why);
  if (!dout || !dq || !dk || !dv || !workspace)
    return fail(PRISM_ERR_ARG, "null tensor or workspace");
  if ((uintptr_t)workspace % 256 || ((uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk |
                                     (uintptr_t)dv) % 16)
    return fail(PRISM_ERR_ARG, "workspace must be 256-byte aligned, dout, dq, dk, dv "
                               "16-byte aligned");
  Layout L = make_layout(d);
  if (workspace_bytes < L.total) return fail(PRISM_ERR_WORKSPACE, "workspace too small");
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto it = g_ws.find((uintptr_t)workspace);
    if (it == g_ws.end() || !same_config(it->second.cfg, *cfg))
      return fail(PRISM_ERR_STATE, "prism_attn_bwd: no prism_plan of this configuration on "
                                   "this workspace");
    if (it->second.fwd_gen != it->second.plan_gen)
      return fail(PRISM_ERR_STATE, "prism_attn_bwd: prism_attn_fwd has not run on this "
                                   "workspace since its last prism_plan");
  }
  Scales sc = scales_of(cfg, d);
  return launched(launch_attn_bwd(d, sc.softmax, (uint8_t *)workspace, L, dout, dq, dk, dv,
                                  (hipStream_t)stream),
                  "attention backward");
}

prism_status prism_forward_static(const prism_config *cfg, const void *q, const void *k,
                                  const void *v, int64_t tok_stride, int64_t head_stride,
                                  const float *a2v_norm, void *o, float *lse, void *stream) {
  Dims d;
  const char *why;
  prism_status st = check_config(cfg, &d, &why);
  if (st != PRISM_OK) return fail(st, why);
  if (!q || !k || !v || !o || !lse) return fail(PRISM_ERR_ARG, "null tensor");
  const size_t need = make_layout(d).total;
  if (need > kScratchBytes)
    return fail(PRISM_ERR_WORKSPACE,
                "prism_forward_static: this configuration needs " + std::to_string(need) +
                    " bytes of workspace, more than the " + std::to_string(kScratchBytes) +
                    "-byte static scratch (use prism_plan and prism_attn_fwd with a "
                    "workspace)");
  int dev = 0;
  if ((st = launched(hipGetDevice(&dev), "prism_forward_static"))) return st;
  void *ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
      if ((st = launched(hipGetSymbolAddress(&ws, HIP_SYMBOL(scratch)), "scratch address")))
        return st;
      g_scratch_ptr[dev] = ws;
    } else {
      ws = it->second;
    }
  }
  // the plan fills every array the forward reads (flags and maxima are cleared by the
  // plan itself), so nothing of the previous call's contents needs clearing
  if ((st = prism_plan(cfg, q, k, v, tok_stride, head_stride, a2v_norm, ws, kScratchBytes,
                       stream)))
    return st;
  return prism_attn_fwd(cfg, ws, kScratchBytes, o, lse, stream);
}

const char *prism_status_string(int status) {
  switch (status) {
    case PRISM_OK: return "ok";
    case PRISM_ERR_ARG: return "invalid argument";
    case PRISM_ERR_UNSUPPORTED: return "unsupported configuration";
    case PRISM_ERR_WORKSPACE: return "workspace too small";
    case PRISM_ERR_HIP: return "HIP launch failure";
    case PRISM_ERR_STATE: return "call out of order for this workspace";
    case PRISM_ERR_RANGE: return "a head's status flags are set";
    default: return "unknown status";
  }
}

const char *prism_last_error(void) { return g_last_error.c_str(); }

prism_status prism_check_flags(const prism_config *cfg, const void *workspace, uint32_t *flags,
                               void *stream) {
  Dims d;
  const char *why;
  prism_status st = check_config(cfg, &d, &why);
  if (st != PRISM_OK) return fail(st, why);
  if (!workspace) return fail(PRISM_ERR_ARG, "null workspace");
  const Layout L = make_layout(d);
  std::vector<uint32_t> host(d.heads);
  hipStream_t s = (hipStream_t)stream;
  if ((st = launched(hipMemcpyAsync(host.data(), (const uint8_t *)workspace + L.pub.flags,
                                    sizeof(uint32_t) * d.heads, hipMemcpyDeviceToHost, s),
                     "flags copy")))
    return st;
  if ((st = launched(hipStreamSynchronize(s), "flags copy"))) return st;
  uint32_t any = 0;
  for (int h = 0; h < d.heads; ++h) {
    any |= host[h];
    if (flags) flags[h] = host[h];
  }
  if (any) {
    std::string msg = "flags set:";
    if (any & PRISM_FLAG_QKV_RANGE) msg += " q/k/v outside the float16 range;";
    if (any & PRISM_FLAG_SELECTION_OVERFLOW) msg += " selection exceeds max_pairs;";
    if (any & PRISM_FLAG_DOUT_RANGE) msg += " dout outside the float16 range;";
    if (any & PRISM_FLAG_DS_RANGE) msg += " dS bound reaches the float16 range;";
    return fail(PRISM_ERR_RANGE, msg);
  }
  return PRISM_OK;
}

prism_status prism_trace_enable(int on) {
  std::lock_guard<std::mutex> lk(g_trace_mu);
  drop_records();
  g_trace_on = on != 0;
  return PRISM_OK;
}

prism_status prism_trace_read(double *ms, int *calls) {
  std::lock_guard<std::mutex> lk(g_trace_mu);
  if (ms)
    for (int i = 0; i < PRISM_STAGE_COUNT; ++i) ms[i] = 0.0;
  if (calls)
    for (int i = 0; i < PRISM_STAGE_COUNT; ++i) calls[i] = 0;
  prism_status st = PRISM_OK;
  for (auto &r : g_records) {
    float t = 0.f;
    if (hipEventSynchronize(r.end) != hipSuccess ||
        hipEventElapsedTime(&t, r.start, r.end) != hipSuccess) {
      st = fail(PRISM_ERR_HIP, "trace event query failed");
      continue;
    }
    if (ms) ms[r.stage] += t;
    if (calls) calls[r.stage] += 1;
  }
  drop_records();
  return st;
}

const char *prism_stage_name(int stage) {
  static const char *names[PRISM_STAGE_COUNT] = {
      "audio_stats", "zone_stats", "quantize", "gather", "tiles", "scores",
      "select",      "attn_fwd",   "bwd_prep", "bwd_dkdv", "bwd_dq"};
  return stage >= 0 && stage < PRISM_STAGE_COUNT ? names[stage] : "unknown";
}

prism_status prism_a2v_norm(const void *x, int64_t n_tokens, int channels, int64_t ld,
                            int dtype, float *a2v_norm, void *stream) {
  if (!x || !a2v_norm) return fail(PRISM_ERR_ARG, "null tensor");
  if (n_tokens <= 0 || channels <= 0 || ld < channels)
    return fail(PRISM_ERR_ARG, "n_tokens and channels must be positive, ld >= channels");
  if (dtype != PRISM_F32 && dtype != PRISM_BF16)
    return fail(PRISM_ERR_UNSUPPORTED, "dtype must be PRISM_F32 or PRISM_BF16");
  const int vpc = dtype == PRISM_BF16 ? 8 : 4;
  if (ld % vpc || ((uintptr_t)x) % 16)
    return fail(PRISM_ERR_ARG, "rows must start on 16-byte boundaries (x aligned, ld * size "
                               "a multiple of 16)");
  if ((n_tokens + 3) / 4 > 0x7fffffffLL) return fail(PRISM_ERR_UNSUPPORTED, "too many tokens");
  return launched(prism::launch_a2v_norm(x, n_tokens, channels, ld, dtype, a2v_norm,
                                         (hipStream_t)stream),
                  "a2v norm");
}

}  // extern "C"
