// Host side of the C ABI declared in include/cdrge.h: configuration checks, workspace plan,
// kernel launch order and diagnostics. All work is enqueued on the caller's stream; the library
// never allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "cdrge.h"
#include "kernels_bf16.h"
#include "kernels_common.h"
#include "kernels_f32.h"
#include "kernels_f32_sliced.h"
#include "kernels_gates_bf16.h"
#include "kernels_update.h"
#include "philox.h"

using namespace cdrge;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxProbes = 1024;
constexpr int64_t kMaxF32LdsBytes = 128 * 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Nearest bf16 to x (ties to even), as a float. x is finite.
float round_bf16_host(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  float r;
  std::memcpy(&r, &u, 4);
  return r;
}

// The probe radius the kernels apply: eps, or bf16(eps) for the exact-perturbation bf16 model,
// whose perturbation enters the matrix products as the bf16 operand eps' P.
float probe_radius(const cdrge_config& c) {
  return c.dtype == CDRGE_BF16_EXACT ? round_bf16_host(c.eps) : c.eps;
}

// Text of the last device-side failure seen by this thread (for cdrge_last_error_detail).
thread_local char g_last_error[256] = "";

cdrge_status device_error(const char* what, hipError_t e) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e),
                static_cast<int>(e));
  return CDRGE_ERR_DEVICE;
}

#define CDRGE_HIP(call)                                          \
  do {                                                           \
    const hipError_t _e = (call);                                \
    if (_e != hipSuccess) return device_error(#call, _e);        \
  } while (0)

struct TensorDesc {
  uint32_t id;
  int64_t off, rows, cols;
};

struct Plan {
  cdrge_config cfg;
  int L, V, E, H, B, T, K, P;
  int64_t d;
  std::vector<TensorDesc> tensors;  // index == tensor id
  size_t off_flags, off_seeds, off_seq, off_emb_m, off_bias_m, off_bout_m, off_x0, off_h, off_c, total;
  int64_t ncols_pad, n_tiles;  // bf16: padded column count of the activation buffers; gate tiles per chunk
  std::vector<size_t> off_wp, off_wm;  // per tensor id (bf16 matrices only)
  std::vector<size_t> off_sg;          // per tensor id (W_ih, W_hh; fp32 also W_out): sign words of a chunk
  std::vector<size_t> off_wt;          // per tensor id (fp32 W_ih, W_hh, W_out): k-major copy W^T
  std::vector<size_t> off_wtile;       // per tensor id (bf16 W_ih, W_hh): tile-major copy for the gate kernel
  int f32_g, f32_nb, f32_threads;      // fp32: pairs and sequences per workgroup, threads
  int ce_slices, ce_kper;              // bf16 logits: K slices (1 = fused) and 32-wide chunks per slice
  bool f32_sliced;                     // fp32: one launch per (layer, t) on row slices (kernels_f32_sliced.h)
  int64_t ncp32;                       // fp32 sliced: column count of a full chunk rounded up to 64
  size_t off_h32, off_c32, off_zp32, off_emb32, off_bias32, off_bout32;  // fp32 sliced state and tables
  size_t off_zpart;                    // bf16 logits: partial logits when split
};

bool basic_valid(const cdrge_config* c) {
  if (!c || c->abi_version != CDRGE_ABI_VERSION) return false;
  if (c->n_layers < 1 || c->vocab < 2 || c->embed < 1 || c->hidden < 1 || c->batch < 1 ||
      c->seq_len < 1 || c->n_probes < 1 || c->probes_per_chunk < 0)
    return false;
  if (c->dtype != CDRGE_F32 && c->dtype != CDRGE_BF16 && c->dtype != CDRGE_BF16_EXACT) return false;
  if (!std::isfinite(c->eps) || !(c->eps > 0.f) || !std::isfinite(c->lr) || c->lr < 0.f) return false;
  return true;
}

int64_t param_count(const cdrge_config* c) {
  const int64_t V = c->vocab, E = c->embed, H = c->hidden;
  int64_t d = V * E + V * H + V;
  for (int l = 0; l < c->n_layers; ++l) d += 4 * H * ((l == 0) ? E : H) + 4 * H * H + 4 * H;
  return d;
}

// fp32 configurations with several sequences per model and enough (model, sequence) columns per
// chunk to fill row-sliced launches (and widths that fit their 32-wide K chunks) run on
// k_lstm_f32_sliced; the others keep the persistent kernel, whose per-model state fits in LDS.
// With one sequence per model (the fixed-batch overfit shape) the persistent kernel measured
// faster: 3.55 against 5.44 ms per step at 1,024 models, H = 256, T = 100 (2.85 ms since).
bool f32_sliced_ok(const cdrge_config* c, int P) {
  return c->dtype == CDRGE_F32 && c->embed % 32 == 0 && c->hidden % 32 == 0 && c->vocab <= kSlMaxV &&
         c->batch >= 8 && int64_t(2) * P * c->batch >= 256 && int64_t(2) * P * c->batch < (int64_t(1) << 30) &&
         c->n_layers <= kF32MaxLayers;
}

cdrge_status supported(const cdrge_config* c) {
  if (c->n_probes > kMaxProbes) return CDRGE_ERR_UNSUPPORTED;
  const int64_t d = param_count(c);
  if (d >= (int64_t(1) << 40)) return CDRGE_ERR_UNSUPPORTED;
  if (int64_t(c->batch) * (c->seq_len + 1) >= (int64_t(1) << 31)) return CDRGE_ERR_UNSUPPORTED;
  const int P = (c->probes_per_chunk == 0 || c->probes_per_chunk > c->n_probes) ? c->n_probes
                                                                               : c->probes_per_chunk;
  if (c->dtype == CDRGE_F32) {
    if (c->n_layers > kF32MaxLayers) return CDRGE_ERR_UNSUPPORTED;
    if (c->hidden > (1 << 16) || c->embed > (1 << 16) || c->vocab > (1 << 16)) return CDRGE_ERR_UNSUPPORTED;
    if (!f32_sliced_ok(c, P)) {
      const int nb = f32_nb(c->batch);
      const F32Lds lay = f32_lds_layout(c->n_layers, c->vocab, c->embed, c->hidden, f32_g(nb, P), nb,
                                        f32_threads(c->hidden));
      if (int64_t(4) * lay.total > kMaxF32LdsBytes) return CDRGE_ERR_UNSUPPORTED;
    }
    const int64_t maxdim = c->embed > c->hidden ? c->embed : c->hidden;
    if (int64_t(4) * c->hidden * maxdim >= (int64_t(1) << 31)) return CDRGE_ERR_UNSUPPORTED;
  } else {
    if (c->embed % 32 != 0 || c->hidden % kUnitsPerTile != 0 || c->vocab > kCeRows)
      return CDRGE_ERR_UNSUPPORTED;
    const int64_t maxdim = c->embed > c->hidden ? c->embed : c->hidden;
    if ((int64_t(2) * P * c->batch + kTileCols) * maxdim >= (int64_t(1) << 31)) return CDRGE_ERR_UNSUPPORTED;
    if (int64_t(2) * P * c->vocab * c->embed >= (int64_t(1) << 31)) return CDRGE_ERR_UNSUPPORTED;
    if (int64_t(4) * c->hidden * (c->embed > c->hidden ? c->embed : c->hidden) >= (int64_t(1) << 31))
      return CDRGE_ERR_UNSUPPORTED;
    if (P > 65535) return CDRGE_ERR_UNSUPPORTED;
  }
  return CDRGE_OK;
}

Plan make_plan(const cdrge_config* c) {
  Plan p;
  p.cfg = *c;
  p.L = c->n_layers;
  p.V = c->vocab;
  p.E = c->embed;
  p.H = c->hidden;
  p.B = c->batch;
  p.T = c->seq_len;
  p.K = c->n_probes;
  p.P = (c->probes_per_chunk == 0 || c->probes_per_chunk > c->n_probes) ? c->n_probes : c->probes_per_chunk;
  int64_t off = 0;
  auto add = [&](uint32_t id, int64_t rows, int64_t cols) {
    p.tensors.push_back(TensorDesc{id, off, rows, cols});
    off += rows * cols;
  };
  add(0, p.V, p.E);
  for (int l = 0; l < p.L; ++l) {
    add(1 + 3 * l, 4 * int64_t(p.H), (l == 0) ? p.E : p.H);
    add(2 + 3 * l, 4 * int64_t(p.H), p.H);
    add(3 + 3 * l, 1, 4 * int64_t(p.H));
  }
  add(1 + 3 * p.L, p.V, p.H);
  add(2 + 3 * p.L, 1, p.V);
  p.d = off;

  const int64_t models = 2 * int64_t(p.P);
  const int64_t ncols = models * p.B;
  size_t w = 0;
  auto region = [&](size_t bytes) {
    const size_t at = w;
    w = align_up(w + bytes);
    return at;
  };
  p.off_flags = region(256);
  p.off_seeds = region(sizeof(uint64_t) * p.K);
  p.off_seq = region(sizeof(float) * models * p.B);
  p.off_wp.assign(p.tensors.size(), 0);
  p.off_wm.assign(p.tensors.size(), 0);
  p.off_sg.assign(p.tensors.size(), 0);
  p.off_wt.assign(p.tensors.size(), 0);
  p.off_wtile.assign(p.tensors.size(), 0);
  p.ce_slices = 1;
  p.ce_kper = 0;
  p.off_zpart = 0;
  p.f32_nb = f32_nb(p.B);
  p.f32_g = f32_g(p.f32_nb, p.P);
  p.f32_threads = f32_threads(p.H);
  p.f32_sliced = f32_sliced_ok(c, p.P);
  p.ncp32 = (ncols + kSlCols - 1) / kSlCols * kSlCols;
  p.off_h32 = p.off_c32 = p.off_zp32 = p.off_emb32 = p.off_bias32 = p.off_bout32 = 0;
  p.off_emb_m = p.off_bias_m = p.off_bout_m = p.off_x0 = p.off_h = p.off_c = 0;
  p.ncols_pad = ncols + kTileCols;
  p.n_tiles = int64_t(p.H / kUnitsPerTile) * ((p.B + kTileCols - 1) / kTileCols) * p.P;
  if (c->dtype != CDRGE_F32) {
    for (const TensorDesc& t : p.tensors) {
      if (t.id != static_cast<uint32_t>(1 + 3 * p.L)) continue;  // W_out: candidates for the logits kernel
      p.off_wp[t.id] = region(sizeof(uint16_t) * t.rows * t.cols);
      p.off_wm[t.id] = region(sizeof(uint16_t) * t.rows * t.cols);
    }
    for (int l = 0; l < p.L; ++l)
      for (const TensorDesc& t : {p.tensors[1 + 3 * l], p.tensors[2 + 3 * l]}) {
        p.off_sg[t.id] = region(sizeof(uint32_t) * p.P * t.rows * (t.cols / 32));
        p.off_wtile[t.id] = region(sizeof(uint16_t) * t.rows * t.cols);
      }
    p.off_emb_m = region(sizeof(uint16_t) * models * p.V * p.E);
    p.off_bias_m = region(sizeof(float) * models * p.L * 4 * p.H);
    p.off_bout_m = region(sizeof(float) * models * kCeRows);
    p.off_x0 = region(sizeof(uint16_t) * p.ncols_pad * p.E);
    p.off_h = region(sizeof(uint16_t) * int64_t(p.L) * 2 * p.ncols_pad * p.H);
    p.off_c = region(sizeof(float) * int64_t(p.L) * p.n_tiles * kGateThreads * 32);
    // Logits: split the reduction over H when column blocks x pairs would leave most CUs idle.
    const int ce_wgs = ((p.B + kCeCols - 1) / kCeCols) * p.P;
    const int nch = p.H / kKChunk;
    int slices = ce_wgs >= kCeTargetWorkgroups ? 1 : (kCeTargetWorkgroups + ce_wgs - 1) / ce_wgs;
    slices = std::max(1, std::min(slices, nch / 4));
    p.ce_kper = ((nch + slices - 1) / slices + 3) / 4 * 4;
    p.ce_slices = (nch + p.ce_kper - 1) / p.ce_kper;
    if (p.ce_slices > 1) p.off_zpart = region(sizeof(float) * p.ce_slices * models * p.B * kCeRows);
  } else {
    for (int l = 0; l <= p.L; ++l) {
      const std::initializer_list<TensorDesc> mats =
          (l < p.L) ? std::initializer_list<TensorDesc>{p.tensors[1 + 3 * l], p.tensors[2 + 3 * l]}
                    : std::initializer_list<TensorDesc>{p.tensors[1 + 3 * p.L]};
      for (const TensorDesc& t : mats) {
        p.off_wt[t.id] = region(sizeof(float) * t.rows * t.cols);
        p.off_sg[t.id] = region(sizeof(uint32_t) * p.P * t.rows * ((t.cols + 31) / 32));
      }
    }
    if (p.f32_sliced) {
      const int64_t ncp = p.ncp32;
      p.off_h32 = region(sizeof(float) * int64_t(p.L) * 2 * p.H * ncp);
      p.off_c32 = region(sizeof(float) * int64_t(p.L) * p.H * ncp);
      p.off_zp32 = region(sizeof(float) * int64_t(p.H / kSlUnits) * p.V * ncp);
      p.off_emb32 = region(sizeof(float) * models * p.V * p.E);
      p.off_bias32 = region(sizeof(float) * models * p.L * 4 * p.H);
      p.off_bout32 = region(sizeof(float) * models * p.V);
    }
  }
  p.total = w;
  return p;
}

__global__ void k_set_u32(uint32_t* p, uint32_t v) { *p = v; }

}  // namespace

namespace {

// k_update_perm instance for G = ceil(K / 8) groups of 8 probes (K <= 64)
template <int kG>
void launch_update_perm_g(dim3 grid, size_t lds, hipStream_t s, uint16_t* theta, const UpdTensors& ut,
                          const uint64_t* seeds, const float* losses, int K, float coef, uint32_t* flags) {
  hipLaunchKernelGGL(k_update_perm<kG>, grid, dim3(kUpdPermThreads), lds, s, theta, ut, seeds, losses, K, coef, flags);
}

void launch_update_perm(int G, dim3 grid, size_t lds, hipStream_t s, uint16_t* theta, const UpdTensors& ut,
                        const uint64_t* seeds, const float* losses, int K, float coef, uint32_t* flags) {
  switch (G) {
    case 1: return launch_update_perm_g<1>(grid, lds, s, theta, ut, seeds, losses, K, coef, flags);
    case 2: return launch_update_perm_g<2>(grid, lds, s, theta, ut, seeds, losses, K, coef, flags);
    case 3: return launch_update_perm_g<3>(grid, lds, s, theta, ut, seeds, losses, K, coef, flags);
    case 4: return launch_update_perm_g<4>(grid, lds, s, theta, ut, seeds, losses, K, coef, flags);
    case 5: return launch_update_perm_g<5>(grid, lds, s, theta, ut, seeds, losses, K, coef, flags);
    case 6: return launch_update_perm_g<6>(grid, lds, s, theta, ut, seeds, losses, K, coef, flags);
    case 7: return launch_update_perm_g<7>(grid, lds, s, theta, ut, seeds, losses, K, coef, flags);
    default: return launch_update_perm_g<8>(grid, lds, s, theta, ut, seeds, losses, K, coef, flags);
  }
}

const void* update_perm_kernel(int G) {
  switch (G) {
    case 1: return reinterpret_cast<const void*>(k_update_perm<1>);
    case 2: return reinterpret_cast<const void*>(k_update_perm<2>);
    case 3: return reinterpret_cast<const void*>(k_update_perm<3>);
    case 4: return reinterpret_cast<const void*>(k_update_perm<4>);
    case 5: return reinterpret_cast<const void*>(k_update_perm<5>);
    case 6: return reinterpret_cast<const void*>(k_update_perm<6>);
    case 7: return reinterpret_cast<const void*>(k_update_perm<7>);
    default: return reinterpret_cast<const void*>(k_update_perm<8>);
  }
}

}  // namespace

struct cdrge_ctx {
  Plan plan;
  void* params = nullptr;
  char* ws = nullptr;
  hipStream_t stream = nullptr;
  int device = 0;
  int n_cu = 1;  // compute units of the device
  bool update_perm = false;  // the update runs k_update_perm
  bool timing = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[4];
  std::vector<hipEvent_t> event_pool;
  double total_ms[4] = {0, 0, 0, 0};
  int64_t launches[4] = {0, 0, 0, 0};
  double work[4] = {0, 0, 0, 0};

  template <class T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(ws + off);
  }

  hipEvent_t get_event() {
    if (!event_pool.empty()) {
      hipEvent_t e = event_pool.back();
      event_pool.pop_back();
      return e;
    }
    // Timing-only events: no system-scope fence when an event is recorded. With the default flag
    // every record writes back and invalidates the caches between two kernels, which slowed a
    // timed step by 1-1.5% and started each timed kernel on a cold L2. The elapsed times are read
    // only after the host has synchronised with the stream.
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
  }
};

namespace {

// Runs `launch` on the context's stream, timing it under `kind` when timing is enabled.
template <class F>
cdrge_status timed(cdrge_ctx* ctx, int kind, double work, F&& launch) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (ctx->timing) {
    e0 = ctx->get_event();
    e1 = ctx->get_event();
    if (!e0 || !e1) return device_error("hipEventCreate", hipErrorOutOfMemory);
    CDRGE_HIP(hipEventRecord(e0, ctx->stream));
  }
  launch();
  CDRGE_HIP(hipGetLastError());
  if (ctx->timing) {
    CDRGE_HIP(hipEventRecord(e1, ctx->stream));
    ctx->pending[kind].emplace_back(e0, e1);
  }
  ctx->work[kind] += work;
  return CDRGE_OK;
}

#define CDRGE_TRY(expr)                   \
  do {                                    \
    const cdrge_status _s = (expr);       \
    if (_s != CDRGE_OK) return _s;        \
  } while (0)

// Where the kernels read the input and the target of (sequence b, step t): in[b * in_stride + t]
// and tg[b * tg_stride + t]. The language-model form reads both from tokens [B][T+1] (target =
// next token, all scored); the transduction form takes [B][T] arrays and allows unscored targets.
struct TokenRefs {
  const int32_t* in;
  int in_stride;
  const int32_t* tg;
  int tg_stride;
  int allow_unscored;
};

TokenRefs lm_refs(const int32_t* tokens, int T) { return TokenRefs{tokens, T + 1, tokens + 1, T + 1, 0}; }

// One probe chunk of an fp32 model on the row-sliced kernels: per-model perturbed embeddings and
// biases, then for every timestep one gate launch per layer (the last one also forms the partial
// logits) and one cross-entropy launch. The chunk's sign words are already in place.
cdrge_status enqueue_f32_sliced(cdrge_ctx* ctx, const TokenRefs& tr, int pair0, int pc, float eps) {
  const Plan& p = ctx->plan;
  const hipStream_t s = ctx->stream;
  const float* theta = static_cast<const float*>(ctx->params);
  const uint64_t* seeds = ctx->at<uint64_t>(p.off_seeds);
  float* seq = ctx->at<float>(p.off_seq);
  const int models = 2 * pc;
  const int ncols = models * p.B;
  const int ncp = (ncols + kSlCols - 1) / kSlCols * kSlCols;
  float* emb = ctx->at<float>(p.off_emb32);
  float* bias = ctx->at<float>(p.off_bias32);
  float* bout = ctx->at<float>(p.off_bout32);
  auto model_tensor = [&](const TensorDesc& t, int out_cols, float* out) {
    const int64_t n = int64_t(models) * t.rows * ((t.cols + 31) / 32);
    return timed(ctx, 3, 0.0, [&] {
      hipLaunchKernelGGL(k_model_tensor_f32, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s,
                         theta + t.off, static_cast<int>(t.rows), static_cast<int>(t.cols), t.id, seeds, pair0,
                         models, eps, out_cols, out);
    });
  };
  CDRGE_TRY(model_tensor(p.tensors[0], p.E, emb));
  for (int l = 0; l < p.L; ++l) CDRGE_TRY(model_tensor(p.tensors[3 + 3 * l], p.L * 4 * p.H, bias + int64_t(l) * 4 * p.H));
  CDRGE_TRY(model_tensor(p.tensors[2 + 3 * p.L], p.V, bout));

  float* hbase = ctx->at<float>(p.off_h32);
  float* cbase = ctx->at<float>(p.off_c32);
  float* zp = ctx->at<float>(p.off_zp32);
  auto hbuf = [&](int l, int par) { return hbase + (int64_t(l) * 2 + par) * p.H * ncp; };
  const dim3 grid(static_cast<uint32_t>(p.H / kSlUnits), static_cast<uint32_t>(ncp / kSlCols));
  const TensorDesc& tout = p.tensors[1 + 3 * p.L];
  for (int t = 0; t < p.T; ++t) {
    for (int l = 0; l < p.L; ++l) {
      const TensorDesc& tih = p.tensors[1 + 3 * l];
      const TensorDesc& thh = p.tensors[2 + 3 * l];
      F32SlArgs g;
      g.wt_ih = ctx->at<float>(p.off_wt[tih.id]);
      g.wt_hh = ctx->at<float>(p.off_wt[thh.id]);
      g.sg_ih = ctx->at<uint32_t>(p.off_sg[tih.id]);
      g.sg_hh = ctx->at<uint32_t>(p.off_sg[thh.id]);
      g.bias_m = bias;
      g.x = l > 0 ? hbuf(l - 1, t & 1) : nullptr;
      g.emb_m = emb;
      g.tok = tr.in;
      g.h_prev = hbuf(l, (t + 1) & 1);
      g.h_out = hbuf(l, t & 1);
      g.c = cbase + int64_t(l) * p.H * ncp;
      g.wt_out = ctx->at<float>(p.off_wt[tout.id]);
      g.sg_out = ctx->at<uint32_t>(p.off_sg[tout.id]);
      g.zpart = zp;
      g.tg = tr.tg;
      g.tg_stride = tr.tg_stride;
      g.eps = eps;
      g.in = static_cast<int>(tih.cols);
      g.H = p.H; g.B = p.B; g.V = p.V; g.L = p.L; g.layer = l; g.t = t;
      g.ncols = ncols; g.ncp = ncp; g.pc = pc; g.in_stride = tr.in_stride;
      g.first = t == 0; g.last = l == p.L - 1;
      // the last layer's logits count only when every target is scored: otherwise a column's
      // logits are formed where its target is scored, which the host does not see, and the count
      // keeps the gate products alone
      const double flops = 2.0 * 4 * p.H * (double(tih.cols) + (t > 0 ? p.H : 0)) * ncols +
                           (l == p.L - 1 && !tr.allow_unscored ? 2.0 * p.V * p.H * ncols : 0.0);
      CDRGE_TRY(timed(ctx, 0, flops, [&] {
        if (p.B % 16 == 0)
          hipLaunchKernelGGL(k_lstm_f32_sliced<true>, grid, dim3(kSlThreads), kSlDirLdsBytes, s, g);
        else
          hipLaunchKernelGGL(k_lstm_f32_sliced<false>, grid, dim3(kSlThreads), kSlLdsBytes, s, g);
      }));
    }
    CDRGE_TRY(timed(ctx, 1, 0.0, [&] {
      hipLaunchKernelGGL(k_ce_f32_sliced, dim3(static_cast<uint32_t>((ncols + 3) / 4)), dim3(256), 0, s, zp, bout,
                         tr.tg, tr.tg_stride, t, p.V, p.B, p.H / kSlUnits, ncols, ncp, seq);
    }));
  }
  return CDRGE_OK;
}

cdrge_status enqueue_probe_losses(cdrge_ctx* ctx, const TokenRefs& tr, uint64_t step, float* losses,
                                  float* seq_losses) {
  const Plan& p = ctx->plan;
  const hipStream_t s = ctx->stream;
  uint32_t* flags = ctx->at<uint32_t>(p.off_flags);
  uint64_t* seeds = ctx->at<uint64_t>(p.off_seeds);
  float* seq = ctx->at<float>(p.off_seq);
  const float eps = probe_radius(p.cfg);
  const bool exact = p.cfg.dtype == CDRGE_BF16_EXACT;

  CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
    hipLaunchKernelGGL(k_seeds, dim3((p.K + 255) / 256), dim3(256), 0, s, p.cfg.base_seed, step, p.K, seeds);
  }));
  CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
    hipLaunchKernelGGL(k_check_tokens, dim3(1), dim3(256), 0, s, tr.in, tr.in_stride, tr.tg, tr.tg_stride, p.B,
                       p.T, p.V, tr.allow_unscored, flags);
  }));

  const bool bf16 = p.cfg.dtype != CDRGE_F32;
  if (!bf16) {
    const float* theta = static_cast<const float*>(ctx->params);
    for (const TensorDesc& t : p.tensors) {
      if (p.off_wt[t.id] == 0) continue;  // not a matrix of the fp32 path (offset 0 holds the flags)
      const dim3 grid(static_cast<uint32_t>((t.cols + 31) / 32), static_cast<uint32_t>((t.rows + 31) / 32));
      CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
        hipLaunchKernelGGL(k_transpose_f32, grid, dim3(256), 0, s, theta + t.off, static_cast<int>(t.rows),
                           static_cast<int>(t.cols), ctx->at<float>(p.off_wt[t.id]));
      }));
    }
  }
  if (bf16) {
    const uint16_t* theta = static_cast<const uint16_t*>(ctx->params);
    // tile-major copies of the gate weights, read by every gate launch of this call
    for (int l = 0; l < p.L; ++l)
      for (const TensorDesc& t : {p.tensors[1 + 3 * l], p.tensors[2 + 3 * l]}) {
        const int64_t pieces = t.rows * t.cols / 8;
        const uint32_t blocks = static_cast<uint32_t>(std::min<int64_t>((pieces + 255) / 256, int64_t(1) << 20));
        CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
          hipLaunchKernelGGL(k_tile_gate_weights, dim3(blocks), dim3(256), 0, s, theta + t.off, p.H,
                             static_cast<int>(t.cols), ctx->at<uint16_t>(p.off_wtile[t.id]));
        }));
      }
    for (const TensorDesc& t : p.tensors) {
      // W_out only (the gate kernels form their own); the exact-perturbation model reads W_out
      // itself and needs no candidates
      if (exact || t.id != static_cast<uint32_t>(1 + 3 * p.L)) continue;
      const int64_t n = t.rows * t.cols;
      CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
        hipLaunchKernelGGL(k_pm_table_bf16, dim3(static_cast<uint32_t>((n / 8 + 256) / 256)), dim3(256), 0, s,
                           theta + t.off, n, eps, ctx->at<uint16_t>(p.off_wp[t.id]),
                           ctx->at<uint16_t>(p.off_wm[t.id]));
      }));
    }
  }

  for (int pair0 = 0; pair0 < p.K; pair0 += p.P) {
    const int pc = (p.K - pair0 < p.P) ? (p.K - pair0) : p.P;
    const int models = 2 * pc;
    const int ncols = models * p.B;
    if (!bf16) {
      for (int l = 0; l <= p.L; ++l) {
        const std::initializer_list<TensorDesc> mats =
            (l < p.L) ? std::initializer_list<TensorDesc>{p.tensors[1 + 3 * l], p.tensors[2 + 3 * l]}
                      : std::initializer_list<TensorDesc>{p.tensors[1 + 3 * p.L]};
        for (const TensorDesc& t : mats) {
          const int wpr = static_cast<int>((t.cols + 31) / 32);
          const int64_t n = int64_t(pc) * t.rows * ((wpr + 3) / 4);
          CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
            hipLaunchKernelGGL(k_sign_words, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s, seeds,
                               pair0, pc, t.id, static_cast<int>(t.rows), wpr, ctx->at<uint32_t>(p.off_sg[t.id]));
          }));
        }
      }
      if (p.f32_sliced) {
        CDRGE_TRY(enqueue_f32_sliced(ctx, tr, pair0, pc, eps));
        CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
          hipLaunchKernelGGL(k_loss_reduce, dim3(models), dim3(256), 0, s, seq, p.B, 2 * pair0, flags, losses,
                             seq_losses);
        }));
        continue;
      }
      F32Args m;
      m.theta = static_cast<const float*>(ctx->params);
      m.off_emb = p.tensors[0].off;
      m.off_bout = p.tensors[2 + 3 * p.L].off;
      for (int l = 0; l < kF32MaxLayers; ++l) {
        const bool on = l < p.L;
        m.off_b[l] = on ? p.tensors[3 + 3 * l].off : 0;
        m.wt_ih[l] = on ? ctx->at<float>(p.off_wt[1 + 3 * l]) : nullptr;
        m.wt_hh[l] = on ? ctx->at<float>(p.off_wt[2 + 3 * l]) : nullptr;
        m.sg_ih[l] = on ? ctx->at<uint32_t>(p.off_sg[1 + 3 * l]) : nullptr;
        m.sg_hh[l] = on ? ctx->at<uint32_t>(p.off_sg[2 + 3 * l]) : nullptr;
      }
      m.wt_out = ctx->at<float>(p.off_wt[1 + 3 * p.L]);
      m.sg_out = ctx->at<uint32_t>(p.off_sg[1 + 3 * p.L]);
      m.in = tr.in;
      m.in_stride = tr.in_stride;
      m.tg = tr.tg;
      m.tg_stride = tr.tg_stride;
      m.seeds = seeds;
      m.seq_out = seq;
      m.eps = eps;
      m.L = p.L; m.V = p.V; m.E = p.E; m.H = p.H; m.B = p.B; m.T = p.T;
      m.pair0 = pair0;
      m.pc = pc;
      const int G = p.f32_g, NB = p.f32_nb, NT = p.f32_threads;
      const size_t lds = sizeof(float) * f32_lds_layout(p.L, p.V, p.E, p.H, G, NB, NT).total;
      // Matrix-product flops actually executed: every timestep, except W_hh h at t = 0 (h = 0).
      double per_token = 2.0 * p.V * p.H, first = 0.0;
      for (int l = 0; l < p.L; ++l) {
        per_token += 2.0 * 4 * p.H * (((l == 0) ? p.E : p.H) + p.H);
        first += 2.0 * 4 * p.H * p.H;
      }
      const double flops = (per_token * p.T - first) * double(ncols);
      const dim3 grid(static_cast<uint32_t>((pc + G - 1) / G), static_cast<uint32_t>((p.B + NB - 1) / NB));
      CDRGE_TRY(timed(ctx, 0, flops, [&] {
        hipLaunchKernelGGL(f32_kernel(G, NB), grid, dim3(NT), lds, s, m);
      }));
    } else {
      const uint16_t* theta = static_cast<const uint16_t*>(ctx->params);
      uint16_t* emb_m = ctx->at<uint16_t>(p.off_emb_m);
      float* bias_m = ctx->at<float>(p.off_bias_m);
      float* bout_m = ctx->at<float>(p.off_bout_m);
      // round: the perturbed value is rounded to bf16 (embedding rows always, as activations of
      // the first product; biases unless the probe is added exactly)
      auto small = [&](const TensorDesc& t, int out_cols, uint16_t* ob, float* of, int round) {
        const int groups = static_cast<int>((t.cols + 31) / 32);
        const int64_t n = int64_t(models) * t.rows * groups;
        return timed(ctx, 3, 0.0, [&] {
          hipLaunchKernelGGL(k_model_tensor_bf16, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s,
                             theta + t.off, static_cast<int>(t.rows), static_cast<int>(t.cols), t.id, seeds,
                             pair0, models, eps, out_cols, round, ob, of);
        });
      };
      CDRGE_TRY(small(p.tensors[0], p.E, emb_m, nullptr, 1));
      for (int l = 0; l < p.L; ++l)
        CDRGE_TRY(small(p.tensors[3 + 3 * l], p.L * 4 * p.H, nullptr, bias_m + int64_t(l) * 4 * p.H, !exact));
      CDRGE_TRY(small(p.tensors[2 + 3 * p.L], kCeRows, nullptr, bout_m, !exact));
      for (int l = 0; l < p.L; ++l)
        for (const TensorDesc& t : {p.tensors[1 + 3 * l], p.tensors[2 + 3 * l]}) {
          const int wpr = static_cast<int>(t.cols / 32);
          const int64_t n = int64_t(pc) * t.rows * ((wpr + 3) / 4);
          CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
            hipLaunchKernelGGL(k_sign_words, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s, seeds,
                               pair0, pc, t.id, static_cast<int>(t.rows), wpr, ctx->at<uint32_t>(p.off_sg[t.id]));
          }));
        }

      uint16_t* hbase = ctx->at<uint16_t>(p.off_h);
      uint16_t* x0 = ctx->at<uint16_t>(p.off_x0);
      float* cbase = ctx->at<float>(p.off_c);
      auto hbuf = [&](int l, int par) { return hbase + (int64_t(l) * 2 + par) * p.ncols_pad * p.H; };
      const int n_rt = p.H / kUnitsPerTile;
      const int n_cb = (p.B + kTileCols - 1) / kTileCols;
      const int n_blocks = n_rt * n_cb * pc;
      // The XCD-grouped order takes groups of group_rows row tiles x group_cols column blocks
      // (16 x 2, else 8 x 4), the last row group of each column group shorter when the row tiles
      // do not divide by group_rows, and needs a multiple of 8 workgroups (then the order is a
      // bijection). An XCD's share need not be whole groups: a group may straddle two XCDs and
      // share less in L2. lstm1b (184 row tiles, 1,472 tiles) ran in plain order while whole
      // groups per XCD were required: 2.03 ms per gate launch, 1.92 ms in 8 x 4 groups, 1.88 ms
      // in 16 x 2 groups with a last group of 8 row tiles.
      int group_rows = 0, group_cols = 0;
      for (const int gr : {16, 8}) {
        const int gc = 32 / gr;
        if (n_rt >= gr && (n_cb * pc) % gc == 0 && n_blocks % 8 == 0) {
          group_rows = gr;
          group_cols = gc;
          break;
        }
      }
      const int swizzle = group_rows > 0;
      const dim3 ggrid(n_blocks);
      const dim3 cgrid((p.B + kCeCols - 1) / kCeCols, pc);
      for (int t = 0; t < p.T; ++t) {
        {
          const dim3 xgrid(static_cast<uint32_t>((4 * p.ncols_pad + 255) / 256),
                           static_cast<uint32_t>((p.E / 32 + kGatherChunks - 1) / kGatherChunks));
          CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
            hipLaunchKernelGGL(k_gather_x0, xgrid, dim3(256), 0, s, emb_m, tr.in, tr.in_stride, p.B, t, p.V,
                               p.E, ncols, static_cast<int>(p.ncols_pad), x0);
          }));
        }
        for (int l = 0; l < p.L; ++l) {
          GateArgs g;
          const TensorDesc& tih = p.tensors[1 + 3 * l];
          const TensorDesc& thh = p.tensors[2 + 3 * l];
          g.w_ih = ctx->at<uint16_t>(p.off_wtile[tih.id]);
          g.w_hh = ctx->at<uint16_t>(p.off_wtile[thh.id]);
          g.eps = eps;
          g.sg_ih = ctx->at<uint32_t>(p.off_sg[tih.id]);
          g.sg_hh = ctx->at<uint32_t>(p.off_sg[thh.id]);
          g.x_in = (l == 0) ? x0 : hbuf(l - 1, t & 1);
          g.h_prev = hbuf(l, (t + 1) & 1);
          g.h_out = hbuf(l, t & 1);
          g.c_tile = cbase + int64_t(l) * p.n_tiles * kGateThreads * 32;
          g.bias_m = bias_m;
          g.in = static_cast<int>(tih.cols);
          g.H = p.H; g.B = p.B; g.L = p.L;
          g.ncols_pad = static_cast<int>(p.ncols_pad);
          g.layer = l;
          g.first = (t == 0) ? 1 : 0;
          g.n_row_tiles = n_rt;
          g.n_col_blocks = n_cb;
          g.n_pairs = pc;
          g.swizzle = swizzle;
          g.group_rows = group_rows;
          g.group_cols = group_cols;
          const double flops = 2.0 * 4 * p.H * double(g.in + (g.first ? 0 : p.H)) * ncols;
          // The instance without requests past the end serves short reductions only (char-LM:
          // gate launch -2.4%), where the 3-6 repeated chunks of every tile are a sizeable share;
          // its main loop compiles to another register assignment, which measured 1.5% and 0.6%
          // slower at 256 and 368 chunks. The exact-perturbation kernel keeps one code path (its
          // registers are already full).
          const int nch = (g.in + (g.first ? 0 : p.H)) / kKChunk;
          const bool phased = !exact && nch % 4 == 0 && nch >= 8 && nch <= kPhasedMaxChunks;
          CDRGE_TRY(timed(ctx, 0, flops, [&] {
            if (exact)
              hipLaunchKernelGGL((k_lstm_gates_bf16<true, false>), ggrid, dim3(kGateThreads), kGateLdsBytes, s, g);
            else if (phased)
              hipLaunchKernelGGL((k_lstm_gates_bf16<false, true>), ggrid, dim3(kGateThreads), kGateLdsBytes, s, g);
            else
              hipLaunchKernelGGL((k_lstm_gates_bf16<false, false>), ggrid, dim3(kGateThreads), kGateLdsBytes, s, g);
          }));
        }
        CeArgs ce;
        const TensorDesc& tw = p.tensors[1 + 3 * p.L];
        // exact perturbation: W_out itself (the kernel adds eps' P), else the two candidates
        ce.wp = exact ? theta + tw.off : ctx->at<uint16_t>(p.off_wp[tw.id]);
        ce.wm = exact ? theta + tw.off : ctx->at<uint16_t>(p.off_wm[tw.id]);
        ce.eps = eps;
        ce.h = hbuf(p.L - 1, t & 1);
        ce.bout_m = bout_m;
        ce.tg = tr.tg;
        ce.tg_stride = tr.tg_stride;
        ce.seeds = seeds;
        ce.seq = seq;
        ce.pair0 = pair0;
        ce.H = p.H; ce.B = p.B; ce.V = p.V; ce.T = p.T; ce.t = t;
        ce.ncols_pad = static_cast<int>(p.ncols_pad);
        ce.tensor_wout = tw.id;
        ce.kper = p.ce_kper;
        ce.zpart = p.ce_slices > 1 ? ctx->at<float>(p.off_zpart) : nullptr;
        const double flops = 2.0 * kCeRows * p.H * double(ncols);
        if (p.ce_slices == 1) {
          CDRGE_TRY(timed(ctx, 1, flops, [&] {
            if (exact)
              hipLaunchKernelGGL((k_logits_ce_bf16<false, true>), cgrid, dim3(kCeThreads), kCeLdsBytes, s, ce);
            else
              hipLaunchKernelGGL((k_logits_ce_bf16<false, false>), cgrid, dim3(kCeThreads), kCeLdsBytes, s, ce);
          }));
        } else {
          const dim3 sgrid(cgrid.x, cgrid.y, static_cast<uint32_t>(p.ce_slices));
          CDRGE_TRY(timed(ctx, 1, flops, [&] {
            if (exact)
              hipLaunchKernelGGL((k_logits_ce_bf16<true, true>), sgrid, dim3(kCeThreads), kCeLdsBytes, s, ce);
            else
              hipLaunchKernelGGL((k_logits_ce_bf16<true, false>), sgrid, dim3(kCeThreads), kCeLdsBytes, s, ce);
          }));
          CDRGE_TRY(timed(ctx, 1, 0.0, [&] {
            hipLaunchKernelGGL(k_ce_reduce, dim3(static_cast<uint32_t>((ncols + 3) / 4)), dim3(256), 0, s,
                               ctx->at<float>(p.off_zpart), p.ce_slices, ncols, p.B, p.V, t, bout_m,
                               tr.tg, tr.tg_stride, seq);
          }));
        }
      }
    }
    CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
      hipLaunchKernelGGL(k_loss_reduce, dim3(models), dim3(256), 0, s, seq, p.B, 2 * pair0, flags, losses,
                         seq_losses);
    }));
  }
  return CDRGE_OK;
}

// The permute-addressed update takes bf16 parameters, K <= 64, all tensors in one launch and
// 32-bit segment indices within a tensor.
bool update_perm_ok(const Plan& p) {
  if (p.cfg.dtype == CDRGE_F32 || p.K > kUpdPermMaxProbes ||
      static_cast<int>(p.tensors.size()) > kUpdMaxTensors)
    return false;
  for (const TensorDesc& t : p.tensors)
    if (t.rows * ((t.cols + 127) / 128) >= (int64_t{1} << 31)) return false;
  return true;
}

cdrge_status enqueue_update(cdrge_ctx* ctx, uint64_t step, const float* losses) {
  const Plan& p = ctx->plan;
  const hipStream_t s = ctx->stream;
  uint32_t* flags = ctx->at<uint32_t>(p.off_flags);
  uint64_t* seeds = ctx->at<uint64_t>(p.off_seeds);
  CDRGE_TRY(timed(ctx, 3, 0.0, [&] {
    hipLaunchKernelGGL(k_seeds, dim3((p.K + 255) / 256), dim3(256), 0, s, p.cfg.base_seed, step, p.K, seeds);
  }));
  // eta / (2 K eps) with the radius the probes actually applied
  const float coef = static_cast<float>(static_cast<double>(p.cfg.lr) /
                                        (2.0 * p.K * static_cast<double>(probe_radius(p.cfg))));
  const bool bf16 = p.cfg.dtype != CDRGE_F32;
  const size_t esz = bf16 ? 2 : 4;
  if (p.K <= kUpdLutMaxProbes && static_cast<int>(p.tensors.size()) <= kUpdMaxTensors) {
    // all tensors in one launch (tensor ids are their positions in the flat layout)
    UpdTensors ut{};
    int64_t segs = 0;
    ut.n = static_cast<int>(p.tensors.size());
    for (int i = 0; i < ut.n; ++i) {
      const TensorDesc& t = p.tensors[i];
      segs += t.rows * ((t.cols + 127) / 128);
      ut.seg_end[i] = segs;
      ut.off[i] = t.off;
      ut.rows[i] = static_cast<int>(t.rows);
      ut.cols[i] = static_cast<int>(t.cols);
    }
    const double bytes = 2.0 * double(p.d) * esz;
    void* th = ctx->params;
    if (ctx->update_perm) {
      // one resident workgroup of 1,024 threads per compute unit, striding over the segments
      const int64_t need = (segs + kUpdPermThreads / 4 - 1) / (kUpdPermThreads / 4);
      const dim3 pgrid(static_cast<uint32_t>(need < ctx->n_cu ? need : ctx->n_cu));
      const size_t lds = update_perm_bytes(p.K);
      return timed(ctx, 2, bytes, [&] {
        launch_update_perm((p.K + 7) / 8, pgrid, lds, s, static_cast<uint16_t*>(th), ut, seeds, losses, p.K, coef,
                           flags);
      });
    }
    const int64_t blocks = (segs + kUpdLutThreads / 4 - 1) / (kUpdLutThreads / 4);
    const dim3 lgrid(static_cast<uint32_t>(blocks < 4096 ? blocks : 4096));
    const int copies = update_lut_copies(p.K);
    const size_t lds = update_lut_bytes(p.K);
    return timed(ctx, 2, bytes, [&] {
      if (bf16) {
        uint16_t* t = static_cast<uint16_t*>(th);
        if (copies == 4)
          hipLaunchKernelGGL((k_update_lut<uint16_t, 4>), lgrid, dim3(kUpdLutThreads), lds, s, t, ut, seeds, losses, p.K, coef, flags);
        else if (copies == 2)
          hipLaunchKernelGGL((k_update_lut<uint16_t, 2>), lgrid, dim3(kUpdLutThreads), lds, s, t, ut, seeds, losses, p.K, coef, flags);
        else
          hipLaunchKernelGGL((k_update_lut<uint16_t, 1>), lgrid, dim3(kUpdLutThreads), lds, s, t, ut, seeds, losses, p.K, coef, flags);
      } else {
        float* t = static_cast<float*>(th);
        if (copies == 4)
          hipLaunchKernelGGL((k_update_lut<float, 4>), lgrid, dim3(kUpdLutThreads), lds, s, t, ut, seeds, losses, p.K, coef, flags);
        else if (copies == 2)
          hipLaunchKernelGGL((k_update_lut<float, 2>), lgrid, dim3(kUpdLutThreads), lds, s, t, ut, seeds, losses, p.K, coef, flags);
        else
          hipLaunchKernelGGL((k_update_lut<float, 1>), lgrid, dim3(kUpdLutThreads), lds, s, t, ut, seeds, losses, p.K, coef, flags);
      }
    });
  }
  for (const TensorDesc& t : p.tensors) {
    const int64_t segs = t.rows * ((t.cols + 127) / 128);
    const dim3 grid(static_cast<uint32_t>((segs + 15) / 16));
    void* base = static_cast<char*>(ctx->params) + t.off * esz;
    const double bytes = 2.0 * double(t.rows * t.cols) * esz;
    CDRGE_TRY(timed(ctx, 2, bytes, [&] {
      if (bf16)
        hipLaunchKernelGGL(k_update<true>, grid, dim3(kUpdThreads), 0, s, base, static_cast<int>(t.rows),
                           static_cast<int>(t.cols), t.id, seeds, losses, p.K, coef, flags);
      else
        hipLaunchKernelGGL(k_update<false>, grid, dim3(kUpdThreads), 0, s, base, static_cast<int>(t.rows),
                           static_cast<int>(t.cols), t.id, seeds, losses, p.K, coef, flags);
    }));
  }
  return CDRGE_OK;
}

// Picks the update kernel and allows it its table LDS. The permute-addressed kernel addresses
// its tables from LDS address 0, which holds while the kernel has no static LDS (checked here).
hipError_t set_update_lds(cdrge_ctx* ctx, bool bf16) {
  const Plan& p = ctx->plan;
  const int K = p.K;
  ctx->update_perm = false;
  if (update_perm_ok(p)) {
    const void* f = update_perm_kernel((ctx->plan.K + 7) / 8);
    hipFuncAttributes fa{};
    const hipError_t e = hipFuncGetAttributes(&fa, f);
    if (e != hipSuccess) return e;
    if (fa.sharedSizeBytes == 0) {
      ctx->update_perm = true;
      return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 static_cast<int>(update_perm_bytes(K)));
    }
  }
  const int copies = update_lut_copies(K);
  const int bytes = static_cast<int>(update_lut_bytes(K));
  const void* f = nullptr;
  if (bf16)
    f = copies == 4 ? reinterpret_cast<const void*>(k_update_lut<uint16_t, 4>)
                    : (copies == 2 ? reinterpret_cast<const void*>(k_update_lut<uint16_t, 2>)
                                   : reinterpret_cast<const void*>(k_update_lut<uint16_t, 1>));
  else
    f = copies == 4 ? reinterpret_cast<const void*>(k_update_lut<float, 4>)
                    : (copies == 2 ? reinterpret_cast<const void*>(k_update_lut<float, 2>)
                                   : reinterpret_cast<const void*>(k_update_lut<float, 1>));
  return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

cdrge_status init_device(cdrge_ctx* ctx, const cdrge_config* cfg) {
  CDRGE_HIP(hipGetDevice(&ctx->device));
  CDRGE_HIP(hipDeviceGetAttribute(&ctx->n_cu, hipDeviceAttributeMultiprocessorCount, ctx->device));
  if (ctx->n_cu < 1) ctx->n_cu = 1;
  if (cfg->dtype != CDRGE_F32) {
    const bool exact = cfg->dtype == CDRGE_BF16_EXACT;
    for (const void* gate : {exact ? reinterpret_cast<const void*>(k_lstm_gates_bf16<true, false>)
                                   : reinterpret_cast<const void*>(k_lstm_gates_bf16<false, false>),
                             reinterpret_cast<const void*>(k_lstm_gates_bf16<false, true>)})
      CDRGE_HIP(hipFuncSetAttribute(gate, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kGateLdsBytes)));
    CDRGE_HIP(set_update_lds(ctx, true));
  } else {
    const Plan& p = ctx->plan;
    if (p.f32_sliced) {
      // with B a multiple of 16 the direct variant (no tables); otherwise the one whose sign-sum
      // tables are addressed from LDS address 0, which needs a kernel without static LDS
      const bool direct = p.B % 16 == 0;
      const void* f = direct ? reinterpret_cast<const void*>(k_lstm_f32_sliced<true>)
                             : reinterpret_cast<const void*>(k_lstm_f32_sliced<false>);
      hipFuncAttributes fa{};
      CDRGE_HIP(hipFuncGetAttributes(&fa, f));
      if (fa.sharedSizeBytes != 0) return device_error("k_lstm_f32_sliced has static LDS", hipErrorInvalidValue);
      CDRGE_HIP(hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    direct ? kSlDirLdsBytes : kSlLdsBytes));
    } else {
      const int lds = static_cast<int>(
          sizeof(float) * f32_lds_layout(p.L, p.V, p.E, p.H, p.f32_g, p.f32_nb, p.f32_threads).total);
      CDRGE_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(f32_kernel(p.f32_g, p.f32_nb)),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    }
    CDRGE_HIP(set_update_lds(ctx, false));
  }
  uint32_t* flags = ctx->at<uint32_t>(ctx->plan.off_flags);
  hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, ctx->stream, flags, 0u);
  hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, ctx->stream, flags + 1, 0u);
  CDRGE_HIP(hipGetLastError());
  return CDRGE_OK;
}

// The library's own device scratch for cdrge_step_noalloc: the workspace of one configuration
// whose plan fits in kScratchBytes. Each device holds its own copy from module load until the
// process ends. In host code `scratch` names a host-side stand-in, never the device memory: host
// code only ever uses the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Address of this device's scratch, looked up once per device with that device current.
cdrge_status device_scratch(void** out) {
  int dev = 0;
  CDRGE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices) return CDRGE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    CDRGE_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) % kAlign) != 0) return CDRGE_ERR_DEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CDRGE_OK;
}

}  // namespace

extern "C" {

const char* cdrge_last_error_detail(void) { return g_last_error; }

int64_t cdrge_param_count(const cdrge_config* cfg) {
  if (!basic_valid(cfg)) return -1;
  return param_count(cfg);
}

cdrge_status cdrge_check_config(const cdrge_config* cfg) {
  if (!basic_valid(cfg)) return CDRGE_ERR_INVALID_ARG;
  return supported(cfg);
}

cdrge_status cdrge_workspace_bytes(const cdrge_config* cfg, size_t* bytes_out) {
  if (!bytes_out) return CDRGE_ERR_INVALID_ARG;
  const cdrge_status st = cdrge_check_config(cfg);
  if (st != CDRGE_OK) return st;
  *bytes_out = make_plan(cfg).total;
  return CDRGE_OK;
}

cdrge_status cdrge_probe_seeds(const cdrge_config* cfg, uint64_t step, uint64_t* seeds_host) {
  if (!basic_valid(cfg) || !seeds_host) return CDRGE_ERR_INVALID_ARG;
  for (int i = 0; i < cfg->n_probes; ++i) seeds_host[i] = probe_seed(cfg->base_seed, step, static_cast<uint32_t>(i));
  return CDRGE_OK;
}

cdrge_status cdrge_init(cdrge_ctx** ctx_out, const cdrge_config* cfg, void* params, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!ctx_out || !params) return CDRGE_ERR_INVALID_ARG;
  *ctx_out = nullptr;
  const cdrge_status st = cdrge_check_config(cfg);
  if (st != CDRGE_OK) return st;
  Plan plan = make_plan(cfg);
  if (!workspace || workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return CDRGE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(params) % 16) != 0) return CDRGE_ERR_INVALID_ARG;
  cdrge_ctx* ctx = new (std::nothrow) cdrge_ctx();
  if (!ctx) return CDRGE_ERR_INVALID_ARG;
  ctx->plan = std::move(plan);
  ctx->params = params;
  ctx->ws = static_cast<char*>(workspace);
  ctx->stream = static_cast<hipStream_t>(stream);
  const cdrge_status st2 = init_device(ctx, cfg);
  if (st2 != CDRGE_OK) {
    delete ctx;
    return st2;
  }
  *ctx_out = ctx;
  return CDRGE_OK;
}

cdrge_status cdrge_probe_losses(cdrge_ctx* ctx, const int32_t* tokens, uint64_t step, float* losses,
                                float* seq_losses) {
  if (!ctx || !tokens || !losses) return CDRGE_ERR_INVALID_ARG;
  return enqueue_probe_losses(ctx, lm_refs(tokens, ctx->plan.T), step, losses, seq_losses);
}

cdrge_status cdrge_probe_losses_io(cdrge_ctx* ctx, const int32_t* inputs, const int32_t* targets,
                                   uint64_t step, float* losses, float* seq_losses) {
  if (!ctx || !inputs || !targets || !losses) return CDRGE_ERR_INVALID_ARG;
  const TokenRefs tr{inputs, ctx->plan.T, targets, ctx->plan.T, 1};
  return enqueue_probe_losses(ctx, tr, step, losses, seq_losses);
}

cdrge_status cdrge_update(cdrge_ctx* ctx, uint64_t step, const float* losses) {
  if (!ctx || !losses) return CDRGE_ERR_INVALID_ARG;
  return enqueue_update(ctx, step, losses);
}

cdrge_status cdrge_step(cdrge_ctx* ctx, const int32_t* tokens, uint64_t step, float* losses) {
  if (!ctx || !tokens || !losses) return CDRGE_ERR_INVALID_ARG;
  CDRGE_TRY(enqueue_probe_losses(ctx, lm_refs(tokens, ctx->plan.T), step, losses, nullptr));
  return enqueue_update(ctx, step, losses);
}

cdrge_status cdrge_step_io(cdrge_ctx* ctx, const int32_t* inputs, const int32_t* targets, uint64_t step,
                           float* losses) {
  if (!ctx || !inputs || !targets || !losses) return CDRGE_ERR_INVALID_ARG;
  const TokenRefs tr{inputs, ctx->plan.T, targets, ctx->plan.T, 1};
  CDRGE_TRY(enqueue_probe_losses(ctx, tr, step, losses, nullptr));
  return enqueue_update(ctx, step, losses);
}

cdrge_status cdrge_sync_status(cdrge_ctx* ctx) {
  if (!ctx) return CDRGE_ERR_INVALID_ARG;
  CDRGE_HIP(hipStreamSynchronize(ctx->stream));
  uint32_t flags[2] = {0, 0};
  CDRGE_HIP(hipMemcpy(flags, ctx->at<uint32_t>(ctx->plan.off_flags), sizeof(flags), hipMemcpyDeviceToHost));
  if (flags[0]) {
    hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, ctx->stream, ctx->at<uint32_t>(ctx->plan.off_flags), 0u);
    CDRGE_HIP(hipGetLastError());
    CDRGE_HIP(hipStreamSynchronize(ctx->stream));
    return CDRGE_ERR_NONFINITE;
  }
  return CDRGE_OK;
}

void cdrge_destroy(cdrge_ctx* ctx) {
  if (!ctx) return;
  for (auto& v : ctx->pending)
    for (auto& pr : v) {
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
  for (hipEvent_t e : ctx->event_pool) (void)hipEventDestroy(e);
  delete ctx;
}

const char* cdrge_status_string(cdrge_status status) {
  switch (status) {
    case CDRGE_OK: return "CDRGE_OK";
    case CDRGE_ERR_INVALID_ARG: return "CDRGE_ERR_INVALID_ARG";
    case CDRGE_ERR_UNSUPPORTED: return "CDRGE_ERR_UNSUPPORTED";
    case CDRGE_ERR_WORKSPACE: return "CDRGE_ERR_WORKSPACE";
    case CDRGE_ERR_DEVICE: return "CDRGE_ERR_DEVICE";
    case CDRGE_ERR_NONFINITE: return "CDRGE_ERR_NONFINITE";
  }
  return "CDRGE_UNKNOWN_STATUS";
}

cdrge_status cdrge_set_timing(cdrge_ctx* ctx, int enable) {
  if (!ctx) return CDRGE_ERR_INVALID_ARG;
  ctx->timing = enable != 0;
  return CDRGE_OK;
}

cdrge_status cdrge_get_timing(cdrge_ctx* ctx, int kind, double* total_ms, int64_t* launches, int reset) {
  if (!ctx || kind < 0 || kind > 3 || !total_ms || !launches) return CDRGE_ERR_INVALID_ARG;
  CDRGE_HIP(hipStreamSynchronize(ctx->stream));
  for (int k = 0; k < 4; ++k) {
    for (auto& pr : ctx->pending[k]) {
      float ms = 0.f;
      CDRGE_HIP(hipEventElapsedTime(&ms, pr.first, pr.second));
      ctx->total_ms[k] += ms;
      ctx->launches[k] += 1;
      ctx->event_pool.push_back(pr.first);
      ctx->event_pool.push_back(pr.second);
    }
    ctx->pending[k].clear();
  }
  *total_ms = ctx->total_ms[kind];
  *launches = ctx->launches[kind];
  if (reset) {
    for (int k = 0; k < 4; ++k) {
      ctx->total_ms[k] = 0;
      ctx->launches[k] = 0;
      ctx->work[k] = 0;
    }
  }
  return CDRGE_OK;
}

const char* cdrge_timed_kernel(const cdrge_ctx* ctx, int kind) {
  if (!ctx || kind < 0 || kind > 3) return "";
  const Plan& p = ctx->plan;
  const bool f32 = p.cfg.dtype == CDRGE_F32;
  switch (kind) {
    case 0: return !f32 ? "k_lstm_gates_bf16" : (p.f32_sliced ? "k_lstm_f32_sliced" : "k_lstm_f32");
    case 1: return !f32 ? "k_logits_ce_bf16" : (p.f32_sliced ? "k_ce_f32_sliced" : "");
    case 2: return ctx->update_perm ? "k_update_perm"
                                    : (static_cast<int>(p.tensors.size()) > kUpdMaxTensors ? "k_update" : "k_update_lut");
    default: return "";
  }
}

cdrge_status cdrge_get_work(cdrge_ctx* ctx, int kind, double* work) {
  if (!ctx || kind < 0 || kind > 3 || !work) return CDRGE_ERR_INVALID_ARG;
  *work = ctx->work[kind];
  return CDRGE_OK;
}

size_t cdrge_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

cdrge_status cdrge_step_noalloc(const cdrge_config* cfg, void* params, const int32_t* tokens,
                                uint64_t step, float* losses, void* stream) {
  if (!params || !tokens || !losses) return CDRGE_ERR_INVALID_ARG;
  const cdrge_status st = cdrge_check_config(cfg);
  if (st != CDRGE_OK) return st;
  if ((reinterpret_cast<uintptr_t>(params) % 16) != 0) return CDRGE_ERR_INVALID_ARG;
  // a context on the stack, bound to the device's scratch instead of a caller workspace
  cdrge_ctx ctx;
  ctx.plan = make_plan(cfg);
  if (ctx.plan.total > kScratchBytes) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "cdrge_step_noalloc: the configuration needs %zu workspace bytes, the static scratch holds %zu",
                  ctx.plan.total, kScratchBytes);
    return CDRGE_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  CDRGE_TRY(device_scratch(&ws));
  ctx.params = params;
  ctx.ws = static_cast<char*>(ws);
  ctx.stream = static_cast<hipStream_t>(stream);
  CDRGE_TRY(init_device(&ctx, cfg));  // clears the status words the previous call left
  CDRGE_TRY(enqueue_probe_losses(&ctx, lm_refs(tokens, ctx.plan.T), step, losses, nullptr));
  return enqueue_update(&ctx, step, losses);
}

}  // extern "C"
