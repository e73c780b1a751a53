// runtime.hip -- host runtime and C ABI of libgptdecode.so (see include/gd.h).
//
// The decode step is one hipGraph launch (one submission per forward pass:
// "bare-metal-llm", "What it taught me"; "rvllm Metal backend", "You record work,
// then you submit it"). Per-step state (positions, lengths, tokens) lives on the
// device, so a captured step replays without host work beyond the launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "gd.h"
#include "common.h"
#include "linear.h"
#include "attention.h"
#include "misc.h"

// ------------------------------------------------------------------ errors

static thread_local std::string g_err;

static gd_status set_err(gd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

extern "C" const char* gd_last_error(void) { return g_err.c_str(); }

#define HIP_TRY(m, call)                                                                   \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) {                                                                \
      if (m) (m)->poisoned = true;                                                         \
      return set_err(GD_ERR_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, __LINE__); \
    }                                                                                      \
  } while (0)

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
static int iceil(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------- linear planning

struct LinPlan {
  int var, mt, mpad, kc, ksplit, ntw, ntiles, grid;
  size_t lds;
};

static const int kLdsBudget = 48 * 1024;

// variant: 0 auto, 1 VALU GEMV, 2 MFMA
static LinPlan plan_linear(int M, int N, int K, int variant) {
  LinPlan p;
  p.var = variant == 1 ? 0 : variant == 2 ? 1 : (M <= 4 ? 0 : 1);
  p.mpad = p.var == 1 ? (M <= 16 ? 16 : 32) : ((M + 3) & ~3);
  p.mt = p.var == 1 ? p.mpad / 16 : 1;
  int kmax = (kLdsBudget / (p.mpad * 4) - 4) & ~31;
  int K32 = (K + 31) & ~31;
  int ks = iceil(K32, kmax);
  int kc = (iceil(K, ks) + 31) & ~31;
  p.ntiles = iceil(N, GD_TILE_N);
  // spread narrow layers over more workgroups with split-K
  while (p.ntiles * ks < 256) {
    int kc2 = (iceil(K, ks + 1) + 31) & ~31;
    if (kc2 < 128 || kc2 >= kc) break;
    ks++;
    kc = kc2;
  }
  p.kc = kc;
  p.ksplit = iceil(K, kc);
  p.ntw = std::max(1, std::min(16, p.ntiles * p.ksplit / 512));
  p.grid = iceil(p.ntiles, p.ntw) * p.ksplit;
  p.lds = (size_t)p.mpad * (p.kc + 4) * sizeof(float);
  return p;
}

static size_t plan_part_floats(const LinPlan& p, int M) {
  return p.ksplit > 1 ? (size_t)p.ntiles * p.ksplit * M * GD_TILE_N : 0;
}

template <int WT>
static hipError_t launch_linear_wt(const LinPlan& lp, const LinearParams& prm, hipStream_t st) {
  if (lp.var == 0) {
    hipLaunchKernelGGL((k_linear<WT, 0, 1>), dim3(lp.grid), dim3(GD_WG), lp.lds, st, prm);
  } else if (lp.mt == 1) {
    hipLaunchKernelGGL((k_linear<WT, 1, 1>), dim3(lp.grid), dim3(GD_WG), lp.lds, st, prm);
  } else {
    hipLaunchKernelGGL((k_linear<WT, 1, 2>), dim3(lp.grid), dim3(GD_WG), lp.lds, st, prm);
  }
  return hipGetLastError();
}

static hipError_t launch_linear(int wt, const LinPlan& lp, LinearParams prm, hipStream_t st) {
  prm.kc = lp.kc;
  prm.ksplit = lp.ksplit;
  prm.ntw = lp.ntw;
  prm.ntiles = lp.ntiles;
  prm.mpad = lp.mpad;
  return wt == GD_WEIGHT_F32 ? launch_linear_wt<0>(lp, prm, st) : launch_linear_wt<1>(lp, prm, st);
}

// ------------------------------------------------------------------- model

struct LayerOff {
  size_t n1g, n1b, wqkv, bqkv, wo, bo, n2g, n2b, wfc, bfc, wproj, bproj;
};

struct GraphKey {
  int batch;
  const void* tok;
  void* next;
  void* logits;
  bool operator<(const GraphKey& o) const {
    return std::tie(batch, tok, next, logits) < std::tie(o.batch, o.tok, o.next, o.logits);
  }
};

struct gd_model {
  gd_config c;
  hipStream_t stream = nullptr;
  hipStream_t cap_stream = nullptr;
  bool poisoned = false;
  int variant = 0;
  bool use_graph = true;
  int dev = 0;

  // derived shapes
  int qdim, kdim, qkvdim, fcN, hdim, wt;
  int nblk, bsize, max_blocks, nchunk, att_chunk;
  size_t elt;  // bytes per weight element

  // sizes
  size_t w_bytes = 0, kv_bytes = 0, s_bytes = 0;
  size_t part_floats = 0, ctr_ints = 0, head_tiles = 0;

  // bound memory
  char* w = nullptr;
  float* kv = nullptr;
  char* s = nullptr;
  bool bound = false, loaded = false;

  // weight offsets (bytes)
  size_t o_wte = 0, o_wpe = 0, o_nfg = 0, o_nfb = 0, o_head = 0;
  std::vector<LayerOff> L;

  // scratch offsets (bytes)
  size_t o_x, o_qkv, o_attn, o_h, o_part, o_ctr, o_amv, o_ami, o_amc, o_apart, o_actr;
  size_t o_rseq, o_rpos, o_rtok, o_pseq, o_ppos, o_ptok, o_len, o_cap, o_sids, o_table, o_err, o_rope;

  // host mirror
  std::vector<int> len, cap;
  std::vector<int> last_sids;
  int* staging = nullptr;  // pinned
  size_t staging_ints = 0;
  hipEvent_t staging_evt = nullptr;
  bool staging_pending = false;

  std::map<GraphKey, hipGraphExec_t> graphs;

  template <class T>
  T* sp(size_t off) const { return reinterpret_cast<T*>(s + off); }
  template <class T>
  const T* wp(size_t off) const { return reinterpret_cast<const T*>(w + off); }
  const float* wf(size_t off) const { return reinterpret_cast<const float*>(w + off); }
  float* kpool(int l) const { return kv + (size_t)l * layer_kv_floats(); }
  float* vpool(int l) const { return kv + (size_t)(c.n_layer + l) * layer_kv_floats(); }
  size_t layer_kv_floats() const { return (size_t)nblk * c.n_kv_head * bsize * c.head_dim; }
};

static gd_status check_cfg(const gd_config* c) {
  if (!c) return set_err(GD_ERR_INVALID, "config is NULL");
  if (c->arch != GD_ARCH_GPT2 && c->arch != GD_ARCH_LLAMA) return set_err(GD_ERR_INVALID, "bad arch %d", c->arch);
  if (c->n_layer < 1 || c->d_model < 8 || c->n_head < 1 || c->n_kv_head < 1 || c->d_ff < 8 || c->vocab < 1 ||
      c->n_ctx < 1)
    return set_err(GD_ERR_INVALID, "bad model sizes");
  if (c->head_dim != 16 && c->head_dim != 64) return set_err(GD_ERR_INVALID, "head_dim must be 16 or 64");
  if (c->d_model % 8 || c->d_ff % 8) return set_err(GD_ERR_INVALID, "d_model and d_ff must be multiples of 8");
  if (c->arch == GD_ARCH_GPT2 && (c->n_kv_head != c->n_head || c->n_head * c->head_dim != c->d_model))
    return set_err(GD_ERR_INVALID, "GPT-2 arch needs n_kv_head == n_head and n_head*head_dim == d_model");
  if (c->n_head % c->n_kv_head) return set_err(GD_ERR_INVALID, "n_head must be a multiple of n_kv_head");
  int G = c->n_head / c->n_kv_head;
  if (G != 1 && G != 3) return set_err(GD_ERR_INVALID, "query heads per KV head must be 1 or 3");
  if ((c->n_head * c->head_dim) % 8) return set_err(GD_ERR_INVALID, "n_head*head_dim must be a multiple of 8");
  if (c->weight_dtype != GD_WEIGHT_F32 && c->weight_dtype != GD_WEIGHT_BF16)
    return set_err(GD_ERR_INVALID, "bad weight_dtype");
  if (c->max_seqs < 1 || c->max_batch < 1 || c->max_batch > GD_MAX_ROWS)
    return set_err(GD_ERR_INVALID, "max_seqs >= 1 and 1 <= max_batch <= 32 required");
  if (c->kv_block_size < 0 || (c->kv_block_size > 0 && c->kv_num_blocks < 1))
    return set_err(GD_ERR_INVALID, "bad paged cache sizes");
  if (!(c->norm_eps > 0.f)) return set_err(GD_ERR_INVALID, "norm_eps must be > 0");
  return GD_OK;
}

static void layout(gd_model* m) {
  const gd_config& c = m->c;
  const size_t d = c.d_model, ff = c.d_ff, V = c.vocab;
  m->wt = c.weight_dtype;
  m->elt = m->wt == GD_WEIGHT_F32 ? 4 : 2;
  m->qdim = c.n_head * c.head_dim;
  m->kdim = c.n_kv_head * c.head_dim;
  m->qkvdim = m->qdim + 2 * m->kdim;
  m->fcN = c.arch == GD_ARCH_GPT2 ? c.d_ff : 2 * c.d_ff;
  m->hdim = c.d_ff;
  if (c.kv_block_size > 0) {
    m->bsize = c.kv_block_size;
    m->nblk = c.kv_num_blocks;
    m->max_blocks = iceil(c.n_ctx, c.kv_block_size);
  } else {
    m->bsize = c.n_ctx;
    m->nblk = c.max_seqs;
    m->max_blocks = 1;
  }
  m->att_chunk = 64;
  m->nchunk = iceil(c.n_ctx, m->att_chunk);

  // weights
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const size_t e = m->elt;
  m->o_wte = take(V * d * e);
  if (c.arch == GD_ARCH_GPT2) m->o_wpe = take((size_t)c.n_ctx * d * e);
  m->L.resize(c.n_layer);
  for (int l = 0; l < c.n_layer; ++l) {
    LayerOff& t = m->L[l];
    t.n1g = take(d * 4);
    t.n1b = c.arch == GD_ARCH_GPT2 ? take(d * 4) : 0;
    t.wqkv = take((size_t)m->qkvdim * d * e);
    t.bqkv = c.arch == GD_ARCH_GPT2 ? take((size_t)m->qkvdim * 4) : 0;
    t.wo = take(d * m->qdim * e);
    t.bo = c.arch == GD_ARCH_GPT2 ? take(d * 4) : 0;
    t.n2g = take(d * 4);
    t.n2b = c.arch == GD_ARCH_GPT2 ? take(d * 4) : 0;
    t.wfc = take((size_t)m->fcN * d * e);
    t.bfc = c.arch == GD_ARCH_GPT2 ? take(ff * 4) : 0;
    t.wproj = take(d * ff * e);
    t.bproj = c.arch == GD_ARCH_GPT2 ? take(d * 4) : 0;
  }
  m->o_nfg = take(d * 4);
  if (c.arch == GD_ARCH_GPT2) m->o_nfb = take(d * 4);
  else m->o_head = take(V * d * e);
  m->w_bytes = off;

  // KV cache: K pools for all layers, then V pools
  m->kv_bytes = 2 * (size_t)c.n_layer * m->layer_kv_floats() * sizeof(float);

  // split-K partials / counters: the largest need over every linear shape and row count
  struct Shp { int N, K; };
  std::vector<Shp> shapes = {{m->qkvdim, c.d_model}, {c.d_model, m->qdim}, {m->fcN, c.d_model},
                             {c.d_model, c.d_ff}, {c.vocab, c.d_model}};
  m->part_floats = 0;
  m->ctr_ints = 0;
  for (auto& sh : shapes)
    for (int M = 1; M <= GD_MAX_ROWS; ++M)
      for (int v = 1; v <= 2; ++v) {
        LinPlan p = plan_linear(M, sh.N, sh.K, v);
        m->part_floats = std::max(m->part_floats, plan_part_floats(p, M));
        m->ctr_ints = std::max(m->ctr_ints, (size_t)p.ntiles);
      }
  m->head_tiles = iceil(c.vocab, GD_TILE_N);

  // scratch
  off = 0;
  const size_t R = GD_MAX_ROWS;
  m->o_x = take(R * d * 4);
  m->o_qkv = take(R * m->qkvdim * 4);
  m->o_attn = take(R * m->qdim * 4);
  m->o_h = take(R * ff * 4);
  m->o_part = take(m->part_floats * 4);
  m->o_ctr = take(m->ctr_ints * 4);
  m->o_amv = take(m->head_tiles * R * 4);
  m->o_ami = take(m->head_tiles * R * 4);
  m->o_amc = take(4);
  m->o_apart = take(R * c.n_head * m->nchunk * (c.head_dim + 2) * 4);
  m->o_actr = take(R * c.n_kv_head * 4);
  m->o_rseq = take(R * 4);
  m->o_rpos = take(R * 4);
  m->o_rtok = take(R * 4);
  m->o_pseq = take((size_t)c.n_ctx * 4);
  m->o_ppos = take((size_t)c.n_ctx * 4);
  m->o_ptok = take((size_t)c.n_ctx * 4);
  m->o_len = take((size_t)c.max_seqs * 4);
  m->o_cap = take((size_t)c.max_seqs * 4);
  m->o_sids = take(R * 4);
  m->o_table = take((size_t)c.max_seqs * m->max_blocks * 4);
  m->o_err = take(4);
  m->o_rope = c.arch == GD_ARCH_LLAMA ? take((size_t)c.n_ctx * c.head_dim * 4) : 0;
  m->s_bytes = off;
}

extern "C" gd_status gd_create(const gd_config* cfg, void* hip_stream, gd_model** out) {
  if (!out) return set_err(GD_ERR_INVALID, "out is NULL");
  *out = nullptr;
  gd_status st = check_cfg(cfg);
  if (st != GD_OK) return st;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return set_err(GD_ERR_NO_DEVICE, "no HIP device");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return set_err(GD_ERR_NO_DEVICE, "hipGetDevice failed");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return set_err(GD_ERR_NO_DEVICE, "no device properties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return set_err(GD_ERR_NO_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  gd_model* m = new gd_model();
  m->c = *cfg;
  m->dev = dev;
  m->stream = reinterpret_cast<hipStream_t>(hip_stream);
  layout(m);
  if (hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&m->staging_evt, hipEventDisableTiming) != hipSuccess) {
    delete m;
    return set_err(GD_ERR_HIP, "stream/event creation failed");
  }
  m->staging_ints = 3 * (size_t)cfg->n_ctx + 64;
  if (hipHostMalloc(reinterpret_cast<void**>(&m->staging), m->staging_ints * sizeof(int), hipHostMallocDefault) !=
      hipSuccess) {
    (void)hipStreamDestroy(m->cap_stream);
    delete m;
    return set_err(GD_ERR_HIP, "pinned staging allocation failed");
  }
  m->len.assign(cfg->max_seqs, 0);
  m->cap.assign(cfg->max_seqs, cfg->kv_block_size > 0 ? 0 : cfg->n_ctx);
  *out = m;
  return GD_OK;
}

extern "C" void gd_destroy(gd_model* m) {
  if (!m) return;
  if (m->stream) (void)hipStreamSynchronize(m->stream);
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  if (m->staging_evt) (void)hipEventDestroy(m->staging_evt);
  if (m->staging) (void)hipHostFree(m->staging);
  delete m;
}

extern "C" gd_status gd_memory_requirements(const gd_model* m, size_t* wb, size_t* kb, size_t* sb) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (wb) *wb = m->w_bytes;
  if (kb) *kb = m->kv_bytes;
  if (sb) *sb = m->s_bytes;
  return GD_OK;
}

// Waits until the pinned staging buffer is no longer read by an enqueued copy.
static gd_status staging_wait(gd_model* m) {
  if (m->staging_pending) {
    HIP_TRY(m, hipEventSynchronize(m->staging_evt));
    m->staging_pending = false;
  }
  return GD_OK;
}

static gd_status staging_done(gd_model* m) {
  HIP_TRY(m, hipEventRecord(m->staging_evt, m->stream));
  m->staging_pending = true;
  return GD_OK;
}

extern "C" gd_status gd_bind_memory(gd_model* m, void* wdev, void* kvdev, void* sdev) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!wdev || !kvdev || !sdev) return set_err(GD_ERR_INVALID, "NULL device buffer");
  if ((reinterpret_cast<uintptr_t>(wdev) | reinterpret_cast<uintptr_t>(kvdev) | reinterpret_cast<uintptr_t>(sdev)) & 255)
    return set_err(GD_ERR_INVALID, "device buffers must be 256-byte aligned");
  m->w = static_cast<char*>(wdev);
  m->kv = static_cast<float*>(kvdev);
  m->s = static_cast<char*>(sdev);
  HIP_TRY(m, hipMemsetAsync(m->s, 0, m->s_bytes, m->stream));
  const gd_config& c = m->c;
  // sequence capacities and (contiguous cache) identity block tables
  HIP_TRY(m, staging_wait(m) == GD_OK ? hipSuccess : hipErrorUnknown);
  std::vector<int> tab((size_t)c.max_seqs * m->max_blocks, -1);
  if (c.kv_block_size == 0)
    for (int s = 0; s < c.max_seqs; ++s) tab[s] = s;
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_table), tab.data(), tab.size() * 4, hipMemcpyHostToDevice, m->stream));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_cap), m->cap.data(), m->cap.size() * 4, hipMemcpyHostToDevice, m->stream));
  if (c.arch == GD_ARCH_LLAMA) {
    const int hd = c.head_dim, half = hd / 2;
    std::vector<float> cs((size_t)c.n_ctx * hd);
    for (int p = 0; p < c.n_ctx; ++p)
      for (int j = 0; j < half; ++j) {
        double ang = (double)p * std::pow((double)c.rope_theta, -2.0 * j / (double)hd);
        cs[(size_t)p * hd + j] = (float)std::cos(ang);
        cs[(size_t)p * hd + half + j] = (float)std::sin(ang);
      }
    HIP_TRY(m, hipMemcpyAsync(m->sp<float>(m->o_rope), cs.data(), cs.size() * 4, hipMemcpyHostToDevice, m->stream));
  }
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  std::fill(m->len.begin(), m->len.end(), 0);
  m->last_sids.clear();
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  m->graphs.clear();
  m->bound = true;
  m->loaded = false;
  return GD_OK;
}

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void put_mat(const gd_model* m, std::vector<char>& dst, size_t off, const float* src, size_t n) {
  if (m->wt == GD_WEIGHT_F32) {
    memcpy(dst.data() + off, src, n * 4);
  } else {
    uint16_t* d = reinterpret_cast<uint16_t*>(dst.data() + off);
    for (size_t i = 0; i < n; ++i) d[i] = to_bf16(src[i]);
  }
}

static void put_vec(std::vector<char>& dst, size_t off, const float* src, size_t n) {
  memcpy(dst.data() + off, src, n * 4);
}

static size_t canonical_count(const gd_config& c) {
  size_t d = c.d_model, ff = c.d_ff, V = c.vocab;
  size_t hq = (size_t)c.n_head * c.head_dim, hk = (size_t)c.n_kv_head * c.head_dim;
  if (c.arch == GD_ARCH_GPT2)
    return V * d + (size_t)c.n_ctx * d + (size_t)c.n_layer * (2 * d + 3 * d * d + 3 * d + d * d + d + 2 * d + ff * d + ff + d * ff + d) + 2 * d;
  return V * d + (size_t)c.n_layer * (d + hq * d + 2 * hk * d + d * hq + d + 2 * ff * d + d * ff) + d + V * d;
}

extern "C" gd_status gd_load_weights(gd_model* m, const float* hw, size_t n) {
  if (!m || !hw) return set_err(GD_ERR_INVALID, "NULL argument");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  const gd_config& c = m->c;
  if (n != canonical_count(c)) return set_err(GD_ERR_INVALID, "weight count %zu, expected %zu", n, canonical_count(c));
  const size_t d = c.d_model, ff = c.d_ff, V = c.vocab, e = m->elt;
  std::vector<char> buf(m->w_bytes, 0);
  const float* p = hw;
  put_mat(m, buf, m->o_wte, p, V * d);
  p += V * d;
  if (c.arch == GD_ARCH_GPT2) {
    put_mat(m, buf, m->o_wpe, p, (size_t)c.n_ctx * d);
    p += (size_t)c.n_ctx * d;
    for (int l = 0; l < c.n_layer; ++l) {
      const LayerOff& t = m->L[l];
      put_vec(buf, t.n1g, p, d); p += d;
      put_vec(buf, t.n1b, p, d); p += d;
      put_mat(m, buf, t.wqkv, p, 3 * d * d); p += 3 * d * d;
      put_vec(buf, t.bqkv, p, 3 * d); p += 3 * d;
      put_mat(m, buf, t.wo, p, d * d); p += d * d;
      put_vec(buf, t.bo, p, d); p += d;
      put_vec(buf, t.n2g, p, d); p += d;
      put_vec(buf, t.n2b, p, d); p += d;
      put_mat(m, buf, t.wfc, p, ff * d); p += ff * d;
      put_vec(buf, t.bfc, p, ff); p += ff;
      put_mat(m, buf, t.wproj, p, d * ff); p += d * ff;
      put_vec(buf, t.bproj, p, d); p += d;
    }
    put_vec(buf, m->o_nfg, p, d); p += d;
    put_vec(buf, m->o_nfb, p, d); p += d;
  } else {
    const size_t hq = m->qdim, hk = m->kdim;
    for (int l = 0; l < c.n_layer; ++l) {
      const LayerOff& t = m->L[l];
      put_vec(buf, t.n1g, p, d); p += d;
      // fused [w_q; w_k; w_v]
      put_mat(m, buf, t.wqkv, p, hq * d); p += hq * d;
      put_mat(m, buf, t.wqkv + hq * d * e, p, hk * d); p += hk * d;
      put_mat(m, buf, t.wqkv + (hq + hk) * d * e, p, hk * d); p += hk * d;
      put_mat(m, buf, t.wo, p, d * hq); p += d * hq;
      put_vec(buf, t.n2g, p, d); p += d;
      // gate/up interleaved per 16-row tile: rows 8j..8j+7 of gate, then of up
      const float* g = p;
      const float* u = p + ff * d;
      for (size_t j = 0; j < ff / 8; ++j) {
        put_mat(m, buf, t.wfc + (j * 16) * d * e, g + j * 8 * d, 8 * d);
        put_mat(m, buf, t.wfc + (j * 16 + 8) * d * e, u + j * 8 * d, 8 * d);
      }
      p += 2 * ff * d;
      put_mat(m, buf, t.wproj, p, d * ff); p += d * ff;
    }
    put_vec(buf, m->o_nfg, p, d); p += d;
    put_mat(m, buf, m->o_head, p, V * d); p += V * d;
  }
  HIP_TRY(m, hipMemcpyAsync(m->w, buf.data(), buf.size(), hipMemcpyHostToDevice, m->stream));
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  m->loaded = true;
  return GD_OK;
}

extern "C" gd_status gd_set_block_table(gd_model* m, int32_t seq, const int32_t* blocks, int32_t n) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  if (m->c.kv_block_size == 0) return set_err(GD_ERR_STATE, "contiguous cache has no block tables");
  if (seq < 0 || seq >= m->c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  if (n < 0 || n > m->max_blocks || (n > 0 && !blocks)) return set_err(GD_ERR_INVALID, "bad block count %d", n);
  for (int i = 0; i < n; ++i)
    if (blocks[i] < 0 || blocks[i] >= m->nblk) return set_err(GD_ERR_INVALID, "block %d out of range", blocks[i]);
  gd_status st = staging_wait(m);
  if (st != GD_OK) return st;
  int* h = m->staging;
  for (int i = 0; i < m->max_blocks; ++i) h[i] = i < n ? blocks[i] : -1;
  int cp = std::min(n * m->bsize, m->c.n_ctx);
  h[m->max_blocks] = cp;
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_table) + (size_t)seq * m->max_blocks, h, m->max_blocks * 4,
                            hipMemcpyHostToDevice, m->stream));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_cap) + seq, h + m->max_blocks, 4, hipMemcpyHostToDevice, m->stream));
  st = staging_done(m);
  if (st != GD_OK) return st;
  m->cap[seq] = cp;
  return GD_OK;
}

extern "C" gd_status gd_reset_seq(gd_model* m, int32_t seq) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  if (seq < 0 || seq >= m->c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  HIP_TRY(m, hipMemsetAsync(m->sp<int>(m->o_len) + seq, 0, 4, m->stream));
  m->len[seq] = 0;
  return GD_OK;
}

extern "C" gd_status gd_seq_len(const gd_model* m, int32_t seq, int32_t* len) {
  if (!m || !len) return set_err(GD_ERR_INVALID, "NULL argument");
  if (seq < 0 || seq >= m->c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  *len = m->len[seq];
  return GD_OK;
}

extern "C" gd_status gd_set_option(gd_model* m, int32_t opt, int32_t v) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (opt == GD_OPT_LINEAR_VARIANT) {
    if (v < 0 || v > 2) return set_err(GD_ERR_INVALID, "variant must be 0, 1 or 2");
    m->variant = v;
  } else if (opt == GD_OPT_USE_GRAPH) {
    m->use_graph = v != 0;
  } else {
    return set_err(GD_ERR_INVALID, "unknown option %d", opt);
  }
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  m->graphs.clear();
  return GD_OK;
}

extern "C" gd_status gd_device_errors(gd_model* m, int32_t* flags) {
  if (!m || !flags) return set_err(GD_ERR_INVALID, "NULL argument");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  int h = 0;
  HIP_TRY(m, hipMemcpyAsync(&h, m->sp<int>(m->o_err), 4, hipMemcpyDeviceToHost, m->stream));
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  HIP_TRY(m, hipMemsetAsync(m->sp<int>(m->o_err), 0, 4, m->stream));
  *flags = h;
  return GD_OK;
}

// ------------------------------------------------------ forward over rows

// Enqueues the forward pass of M (<= 32) rows with device-resident row metadata.
// If head_out is not NULL, computes logits/argmax for rows [head_row, head_row + head_rows).
static hipError_t enqueue_rows(gd_model* m, hipStream_t st, int M, const int* rseq, const int* rpos,
                               const int* rtok, int head_row, int head_rows, int* head_out, float* logits) {
  const gd_config& c = m->c;
  const int d = c.d_model, ff = c.d_ff;
  float* x = m->sp<float>(m->o_x);
  float* qkv = m->sp<float>(m->o_qkv);
  float* attn = m->sp<float>(m->o_attn);
  float* h = m->sp<float>(m->o_h);
  int* err = m->sp<int>(m->o_err);
  hipError_t e;
  if (m->wt == GD_WEIGHT_F32)
    hipLaunchKernelGGL(k_embed<0>, dim3(M), dim3(GD_WG), 0, st, m->w + m->o_wte,
                       c.arch == GD_ARCH_GPT2 ? (const void*)(m->w + m->o_wpe) : nullptr, c.vocab, c.n_ctx, d, rtok,
                       rpos, x, d, err);
  else
    hipLaunchKernelGGL(k_embed<1>, dim3(M), dim3(GD_WG), 0, st, m->w + m->o_wte,
                       c.arch == GD_ARCH_GPT2 ? (const void*)(m->w + m->o_wpe) : nullptr, c.vocab, c.n_ctx, d, rtok,
                       rpos, x, d, err);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  LinearParams base;
  memset(&base, 0, sizeof(base));
  base.eps = c.norm_eps;
  base.part = m->sp<float>(m->o_part);
  base.ctr = m->sp<int>(m->o_ctr);
  const int nrm = c.arch == GD_ARCH_GPT2 ? 1 : 2;
  const int G = c.n_head / c.n_kv_head;

  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& t = m->L[l];
    // QKV (+ pre-norm, + bias)
    {
      LinearParams p = base;
      p.x = x; p.ldx = d; p.w = m->w + t.wqkv;
      p.bias = t.bqkv ? m->wf(t.bqkv) : nullptr;
      p.norm = nrm; p.ng = m->wf(t.n1g); p.nb = t.n1b ? m->wf(t.n1b) : nullptr;
      p.act = LIN_ACT_NONE; p.y = qkv; p.ldy = m->qkvdim;
      p.M = M; p.N = m->qkvdim; p.K = d;
      if ((e = launch_linear(m->wt, plan_linear(M, p.N, p.K, m->variant), p, st)) != hipSuccess) return e;
    }
    // RoPE + KV append
    hipLaunchKernelGGL(k_rope_append, dim3(M), dim3(GD_WG), 0, st, qkv, m->qkvdim, c.n_head, c.n_kv_head,
                       c.head_dim, c.arch == GD_ARCH_LLAMA ? m->sp<float>(m->o_rope) : (float*)nullptr, c.n_ctx,
                       m->kpool(l), m->vpool(l), m->sp<int>(m->o_table), m->max_blocks, m->bsize, m->nblk, rseq,
                       rpos, err);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // attention
    {
      AttnParams a;
      a.q = qkv; a.ldq = m->qkvdim; a.out = attn; a.ldo = m->qdim;
      a.kc = m->kpool(l); a.vc = m->vpool(l);
      a.table = m->sp<int>(m->o_table); a.max_blocks = m->max_blocks; a.block_size = m->bsize; a.nblk = m->nblk;
      a.Hq = c.n_head; a.Hkv = c.n_kv_head; a.row_seq = rseq; a.row_pos = rpos;
      a.M = M; a.nchunk = m->nchunk; a.chunk = m->att_chunk;
      a.scale = 1.0f / std::sqrt((float)c.head_dim);
      a.part = m->sp<float>(m->o_apart); a.ctr = m->sp<int>(m->o_actr);
      dim3 grid(m->nchunk, c.n_kv_head, M);
      if (c.head_dim == 64 && G == 1) hipLaunchKernelGGL((k_attention<64, 1>), grid, dim3(GD_WG), 0, st, a);
      else if (c.head_dim == 64 && G == 3) hipLaunchKernelGGL((k_attention<64, 3>), grid, dim3(GD_WG), 0, st, a);
      else if (c.head_dim == 16 && G == 1) hipLaunchKernelGGL((k_attention<16, 1>), grid, dim3(GD_WG), 0, st, a);
      else hipLaunchKernelGGL((k_attention<16, 3>), grid, dim3(GD_WG), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // output projection + bias + residual (in place on x)
    {
      LinearParams p = base;
      p.x = attn; p.ldx = m->qdim; p.w = m->w + t.wo;
      p.bias = t.bo ? m->wf(t.bo) : nullptr;
      p.resid = x; p.ldr = d; p.y = x; p.ldy = d;
      p.M = M; p.N = d; p.K = m->qdim;
      if ((e = launch_linear(m->wt, plan_linear(M, p.N, p.K, m->variant), p, st)) != hipSuccess) return e;
    }
    // MLP up: GPT-2 FC + bias + GELU; Llama gate|up + SiLU gate
    {
      LinearParams p = base;
      p.x = x; p.ldx = d; p.w = m->w + t.wfc;
      p.bias = t.bfc ? m->wf(t.bfc) : nullptr;
      p.norm = nrm; p.ng = m->wf(t.n2g); p.nb = t.n2b ? m->wf(t.n2b) : nullptr;
      p.act = c.arch == GD_ARCH_GPT2 ? LIN_ACT_GELU : LIN_ACT_SWIGLU;
      p.y = h; p.ldy = ff;
      p.M = M; p.N = m->fcN; p.K = d;
      if ((e = launch_linear(m->wt, plan_linear(M, p.N, p.K, m->variant), p, st)) != hipSuccess) return e;
    }
    // MLP down + bias + residual
    {
      LinearParams p = base;
      p.x = h; p.ldx = ff; p.w = m->w + t.wproj;
      p.bias = t.bproj ? m->wf(t.bproj) : nullptr;
      p.resid = x; p.ldr = d; p.y = x; p.ldy = d;
      p.M = M; p.N = d; p.K = ff;
      if ((e = launch_linear(m->wt, plan_linear(M, p.N, p.K, m->variant), p, st)) != hipSuccess) return e;
    }
  }
  if (head_out) {
    LinearParams p = base;
    p.x = x + (size_t)head_row * d; p.ldx = d;
    p.w = m->w + (c.arch == GD_ARCH_GPT2 ? m->o_wte : m->o_head);
    p.norm = nrm; p.ng = m->wf(m->o_nfg); p.nb = c.arch == GD_ARCH_GPT2 ? m->wf(m->o_nfb) : nullptr;
    p.act = LIN_ACT_ARGMAX;
    p.M = head_rows; p.N = c.vocab; p.K = d;
    p.am_val = m->sp<float>(m->o_amv); p.am_idx = m->sp<int>(m->o_ami); p.am_ctr = m->sp<int>(m->o_amc);
    p.am_out = head_out; p.logits = logits; p.ldl = c.vocab;
    if ((e = launch_linear(m->wt, plan_linear(head_rows, p.N, p.K, m->variant), p, st)) != hipSuccess) return e;
  }
  return hipSuccess;
}

static gd_status ready(gd_model* m) {
  if (!m) return set_err(GD_ERR_INVALID, "model is NULL");
  if (m->poisoned) return set_err(GD_ERR_HIP, "model is poisoned by an earlier HIP error");
  if (!m->bound) return set_err(GD_ERR_STATE, "memory not bound");
  if (!m->loaded) return set_err(GD_ERR_STATE, "weights not loaded");
  return GD_OK;
}

extern "C" gd_status gd_prefill(gd_model* m, int32_t seq, const int32_t* tokens, int32_t n, int32_t* next_dev,
                                float* logits_dev) {
  gd_status st = ready(m);
  if (st != GD_OK) return st;
  const gd_config& c = m->c;
  if (seq < 0 || seq >= c.max_seqs) return set_err(GD_ERR_INVALID, "seq %d out of range", seq);
  if (!tokens || n < 1) return set_err(GD_ERR_INVALID, "prefill needs at least one token");
  if (!next_dev) return set_err(GD_ERR_INVALID, "next_token_dev is NULL");
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.vocab) return set_err(GD_ERR_INVALID, "token %d out of range at %d", tokens[i], i);
  const int p0 = m->len[seq];
  if (p0 + n > m->cap[seq])
    return set_err(GD_ERR_CTX_FULL, "sequence %d: %d + %d positions exceed capacity %d", seq, p0, n, m->cap[seq]);
  if ((st = staging_wait(m)) != GD_OK) return st;
  int* hs = m->staging;
  int* hp = hs + n;
  int* ht = hs + 2 * n;
  for (int i = 0; i < n; ++i) { hs[i] = seq; hp[i] = p0 + i; ht[i] = tokens[i]; }
  hs[3 * n] = p0 + n;
  hipStream_t s = m->stream;
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_pseq), hs, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_ppos), hp, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_ptok), ht, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_len) + seq, hs + 3 * n, 4, hipMemcpyHostToDevice, s));
  if ((st = staging_done(m)) != GD_OK) return st;
  for (int r0 = 0; r0 < n; r0 += GD_MAX_ROWS) {
    int M = std::min(GD_MAX_ROWS, n - r0);
    bool last = r0 + M == n;
    hipError_t e = enqueue_rows(m, s, M, m->sp<int>(m->o_pseq) + r0, m->sp<int>(m->o_ppos) + r0,
                                m->sp<int>(m->o_ptok) + r0, M - 1, 1, last ? next_dev : nullptr,
                                last ? logits_dev : nullptr);
    if (e != hipSuccess) {
      m->poisoned = true;
      return set_err(GD_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    }
  }
  m->len[seq] = p0 + n;
  return GD_OK;
}

static hipError_t enqueue_decode(gd_model* m, hipStream_t st, int B, const int* tok, int* next, float* logits) {
  hipLaunchKernelGGL(k_setup_decode, dim3(1), dim3(64), 0, st, B, m->sp<int>(m->o_sids), tok, m->sp<int>(m->o_len),
                     m->sp<int>(m->o_cap), m->sp<int>(m->o_rseq), m->sp<int>(m->o_rpos), m->sp<int>(m->o_rtok),
                     m->sp<int>(m->o_err));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return enqueue_rows(m, st, B, m->sp<int>(m->o_rseq), m->sp<int>(m->o_rpos), m->sp<int>(m->o_rtok), 0, B, next,
                      logits);
}

extern "C" gd_status gd_decode_step(gd_model* m, int32_t B, const int32_t* sids, const int32_t* tok_dev,
                                    int32_t* next_dev, float* logits_dev) {
  gd_status st = ready(m);
  if (st != GD_OK) return st;
  const gd_config& c = m->c;
  if (B < 1 || B > c.max_batch) return set_err(GD_ERR_INVALID, "batch %d outside 1..%d", B, c.max_batch);
  if (!sids || !tok_dev || !next_dev) return set_err(GD_ERR_INVALID, "NULL argument");
  for (int b = 0; b < B; ++b) {
    if (sids[b] < 0 || sids[b] >= c.max_seqs) return set_err(GD_ERR_INVALID, "seq id %d out of range", sids[b]);
    for (int b2 = 0; b2 < b; ++b2)
      if (sids[b2] == sids[b]) return set_err(GD_ERR_INVALID, "seq id %d repeated in the batch", sids[b]);
    if (m->len[sids[b]] < 1) return set_err(GD_ERR_STATE, "sequence %d has no prefilled context", sids[b]);
    if (m->len[sids[b]] >= m->cap[sids[b]])
      return set_err(GD_ERR_CTX_FULL, "sequence %d is full (%d positions)", sids[b], m->cap[sids[b]]);
  }
  hipStream_t s = m->stream;
  std::vector<int> want(sids, sids + B);
  if (want != m->last_sids) {
    if ((st = staging_wait(m)) != GD_OK) return st;
    memcpy(m->staging, sids, (size_t)B * 4);
    HIP_TRY(m, hipMemcpyAsync(m->sp<int>(m->o_sids), m->staging, (size_t)B * 4, hipMemcpyHostToDevice, s));
    if ((st = staging_done(m)) != GD_OK) return st;
    m->last_sids = want;
  }
  if (m->use_graph) {
    GraphKey key{B, tok_dev, next_dev, logits_dev};
    auto it = m->graphs.find(key);
    if (it == m->graphs.end()) {
      hipGraph_t g;
      HIP_TRY(m, hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal));
      hipError_t e = enqueue_decode(m, m->cap_stream, B, tok_dev, next_dev, logits_dev);
      hipError_t e2 = hipStreamEndCapture(m->cap_stream, &g);
      if (e != hipSuccess || e2 != hipSuccess) {
        m->poisoned = true;
        return set_err(GD_ERR_HIP, "decode capture failed: %s / %s", hipGetErrorString(e), hipGetErrorString(e2));
      }
      hipGraphExec_t ex;
      hipError_t e3 = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
      (void)hipGraphDestroy(g);
      if (e3 != hipSuccess) {
        m->poisoned = true;
        return set_err(GD_ERR_HIP, "graph instantiate failed: %s", hipGetErrorString(e3));
      }
      it = m->graphs.emplace(key, ex).first;
    }
    HIP_TRY(m, hipGraphLaunch(it->second, s));
  } else {
    hipError_t e = enqueue_decode(m, s, B, tok_dev, next_dev, logits_dev);
    if (e != hipSuccess) {
      m->poisoned = true;
      return set_err(GD_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    }
  }
  for (int b = 0; b < B; ++b) m->len[sids[b]] += 1;
  return GD_OK;
}

// ---------------------------------------------------------------- op level

static gd_status linear_ws(int M, int N, int K, int variant, size_t* bytes, LinPlan* out) {
  if (M < 1 || M > GD_MAX_ROWS || N < 1 || K < 8 || K % 8) return set_err(GD_ERR_INVALID, "bad shape M=%d N=%d K=%d", M, N, K);
  if (variant < 0 || variant > 2) return set_err(GD_ERR_INVALID, "bad variant %d", variant);
  LinPlan p = plan_linear(M, N, K, variant);
  if (out) *out = p;
  *bytes = align_up(plan_part_floats(p, M) * 4, 256) + align_up((size_t)p.ntiles * 4, 256);
  return GD_OK;
}

extern "C" gd_status gd_linear_workspace(int32_t M, int32_t N, int32_t K, int32_t variant, size_t* bytes) {
  if (!bytes) return set_err(GD_ERR_INVALID, "bytes is NULL");
  return linear_ws(M, N, K, variant, bytes, nullptr);
}

extern "C" gd_status gd_linear(const float* x, int32_t ldx, const void* W, int32_t wdt, const float* bias,
                               int32_t norm, const float* ng, const float* nb, float eps, int32_t act,
                               const float* resid, int32_t ldr, float* y, int32_t ldy, int32_t M, int32_t N, int32_t K,
                               int32_t variant, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  LinPlan lp;
  gd_status st = linear_ws(M, N, K, variant, &need, &lp);
  if (st != GD_OK) return st;
  if (!x || !W || !y) return set_err(GD_ERR_INVALID, "NULL argument");
  if (wdt != GD_WEIGHT_F32 && wdt != GD_WEIGHT_BF16) return set_err(GD_ERR_INVALID, "bad weight dtype");
  if (norm < 0 || norm > 2 || (norm && !ng) || (norm == 1 && !nb)) return set_err(GD_ERR_INVALID, "bad norm");
  if (act != GD_ACT_NONE && act != GD_ACT_GELU) return set_err(GD_ERR_INVALID, "bad act");
  if (ldx < K || ldx % 4 || ldy < N || (resid && ldr < N)) return set_err(GD_ERR_INVALID, "bad leading dimensions");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(W)) & 15)
    return set_err(GD_ERR_INVALID, "x and W must be 16-byte aligned");
  if (ws_bytes < need || (need && !ws)) return set_err(GD_ERR_OOM, "workspace %zu < %zu bytes", ws_bytes, need);
  LinearParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.ldx = ldx; p.w = W; p.bias = bias; p.norm = norm; p.ng = ng; p.nb = nb; p.eps = eps;
  p.act = act; p.resid = resid; p.ldr = ldr; p.y = y; p.ldy = ldy; p.M = M; p.N = N; p.K = K;
  p.part = static_cast<float*>(ws);
  p.ctr = reinterpret_cast<int*>(static_cast<char*>(ws) + align_up(plan_part_floats(lp, M) * 4, 256));
  hipError_t e = launch_linear(wdt, lp, p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_err(GD_ERR_HIP, "linear launch failed: %s", hipGetErrorString(e));
  return GD_OK;
}

extern "C" gd_status gd_argmax_workspace(int32_t rows, int32_t vocab, size_t* bytes) {
  if (!bytes || rows < 1 || rows > GD_MAX_ROWS || vocab < 1) return set_err(GD_ERR_INVALID, "bad argmax shape");
  int nch = iceil(vocab, 4096);
  *bytes = 2 * align_up((size_t)rows * nch * 4, 256) + align_up((size_t)rows * 4, 256);
  return GD_OK;
}

extern "C" gd_status gd_argmax(const float* logits, int32_t rows, int32_t vocab, int32_t* out, void* ws,
                               size_t ws_bytes, void* stream) {
  size_t need;
  gd_status st = gd_argmax_workspace(rows, vocab, &need);
  if (st != GD_OK) return st;
  if (!logits || !out || !ws) return set_err(GD_ERR_INVALID, "NULL argument");
  if (ws_bytes < need) return set_err(GD_ERR_OOM, "workspace %zu < %zu bytes", ws_bytes, need);
  int nch = iceil(vocab, 4096);
  char* b = static_cast<char*>(ws);
  float* pv = reinterpret_cast<float*>(b);
  int* pi = reinterpret_cast<int*>(b + align_up((size_t)rows * nch * 4, 256));
  int* ctr = reinterpret_cast<int*>(b + 2 * align_up((size_t)rows * nch * 4, 256));
  hipLaunchKernelGGL(k_argmax_rows, dim3(nch, rows), dim3(GD_WG), 0, reinterpret_cast<hipStream_t>(stream), logits,
                     rows, vocab, nch, pv, pi, ctr, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_err(GD_ERR_HIP, "argmax launch failed: %s", hipGetErrorString(e));
  return GD_OK;
}
