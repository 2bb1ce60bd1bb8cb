// Host engine of the S3-DiT forward behind the C ABI of include/zimg_dit.h.
//
// What it owns: the model's weights on the device in the layout the kernels
// want (bf16 matrices, fp32 vectors, q|k|v fused, w1/w3 interleaved in
// groups of 32 rows, every block's adaLN projection concatenated into one
// matrix), the whole forward workspace (sized at create, never allocated
// inside a forward), the host-built RoPE tables and attention work lists
// (cached per input geometry), and the block schedule.
//
// Row layout of the sequence buffer: all image rows of the batch (sample b
// at b*Npad, Npad = image tokens rounded up to 16), then all caption rows
// (sample b at its own offset, lengths rounded up to 16).  Padding rows
// belong to no attention segment, so they never influence real rows.  The
// noise refiner works on the image rows, the context refiner on the
// caption rows, the joint blocks on all rows ("Z-Image" (AI Toolkit docs),
// Architecture: text and image tokens share one sequence; 2 noise-refiner
// blocks on image tokens, 2 context-refiner blocks on text tokens).
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/zimg_dit.h"
#include "../../include/zimg_ops.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int set_err(int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace

namespace zimg {
int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
}  // namespace zimg

namespace {

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return set_err(ZIMG_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));        \
  } while (0)

// run ``call`` (a hipError_t expression) bracketed by the profiler's events
#define PROFILED(cls, call)                          \
  do {                                               \
    int prc_ = prof_start(cls, s);                   \
    if (prc_) return prc_;                           \
    HIP_TRY(call);                                   \
    prc_ = prof_stop(s);                             \
    if (prc_) return prc_;                           \
  } while (0)

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float bf16_to_f32(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// ------------------------------------------------------------------ manifest

struct ManifestEntry {
  std::string name;
  int ndim;
  int64_t shape[4];
};

struct BlockSpec {
  std::string prefix;
  int stage;      // 0 noise refiner, 1 context refiner, 2 joint
  bool modulated;
};

std::vector<BlockSpec> block_specs(const zimg_dit_config& c) {
  std::vector<BlockSpec> v;
  for (int i = 0; i < c.n_noise_refiner; ++i) v.push_back({"noise_refiner." + std::to_string(i), 0, true});
  for (int i = 0; i < c.n_context_refiner; ++i) v.push_back({"context_refiner." + std::to_string(i), 1, false});
  for (int i = 0; i < c.n_layers; ++i) v.push_back({"layers." + std::to_string(i), 2, true});
  return v;
}

std::vector<ManifestEntry> build_manifest(const zimg_dit_config& c) {
  const int64_t D = c.hidden, F = c.ffn, P = (int64_t)c.patch * c.patch * c.in_channels;
  std::vector<ManifestEntry> m;
  auto add = [&](const std::string& n, std::initializer_list<int64_t> s) {
    ManifestEntry e;
    e.name = n;
    e.ndim = (int)s.size();
    int i = 0;
    for (int64_t v : s) e.shape[i++] = v;
    for (; i < 4; ++i) e.shape[i] = 0;
    m.push_back(e);
  };
  add("t_embedder.mlp.0.weight", {c.t_mid, c.adaln_dim});
  add("t_embedder.mlp.0.bias", {c.t_mid});
  add("t_embedder.mlp.2.weight", {c.adaln_dim, c.t_mid});
  add("t_embedder.mlp.2.bias", {c.adaln_dim});
  add("cap_embedder.0.weight", {c.cap_feat_dim});
  add("cap_embedder.1.weight", {D, c.cap_feat_dim});
  add("cap_embedder.1.bias", {D});
  add("all_x_embedder.2-1.weight", {D, P});
  add("all_x_embedder.2-1.bias", {D});
  add("all_final_layer.2-1.adaLN_modulation.1.weight", {D, c.adaln_dim});
  add("all_final_layer.2-1.adaLN_modulation.1.bias", {D});
  add("all_final_layer.2-1.linear.weight", {P, D});
  add("all_final_layer.2-1.linear.bias", {P});
  add("x_pad_token", {1, D});
  add("cap_pad_token", {1, D});
  for (const auto& b : block_specs(c)) {
    const std::string& p = b.prefix;
    add(p + ".attention.to_q.weight", {D, D});
    add(p + ".attention.to_k.weight", {D, D});
    add(p + ".attention.to_v.weight", {D, D});
    add(p + ".attention.to_out.0.weight", {D, D});
    add(p + ".attention.norm_q.weight", {128});
    add(p + ".attention.norm_k.weight", {128});
    add(p + ".feed_forward.w1.weight", {F, D});
    add(p + ".feed_forward.w2.weight", {D, F});
    add(p + ".feed_forward.w3.weight", {F, D});
    add(p + ".attention_norm1.weight", {D});
    add(p + ".attention_norm2.weight", {D});
    add(p + ".ffn_norm1.weight", {D});
    add(p + ".ffn_norm2.weight", {D});
    if (b.modulated) {
      add(p + ".adaLN_modulation.0.weight", {4 * D, c.adaln_dim});
      add(p + ".adaLN_modulation.0.bias", {4 * D});
    }
  }
  return m;
}

// manifests are cached per config so that entry names stay valid for the
// life of the process; the cache may be reached from several threads (a
// manifest query while another thread creates an engine), hence the lock.
// Entries are never removed, so a returned reference stays valid unlocked.
// (the key is the config's bytes: 25 four-byte fields, no padding)
static_assert(sizeof(zimg_dit_config) == 26 * 4, "zimg_dit_config must have no padding");
const std::vector<ManifestEntry>& cached_manifest(const zimg_dit_config& c) {
  static std::mutex mu;
  static std::map<std::string, std::unique_ptr<std::vector<ManifestEntry>>> cache;
  const std::string key((const char*)&c, sizeof c);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it == cache.end()) it = cache.emplace(key, std::make_unique<std::vector<ManifestEntry>>(build_manifest(c))).first;
  return *it->second;
}

int check_config(const zimg_dit_config* c) {
  if (!c) return set_err(ZIMG_EINVAL, "config is NULL");
  if (c->n_heads <= 0 || c->hidden != c->n_heads * 128)
    return set_err(ZIMG_EUNSUPPORTED, "hidden (%d) must equal n_heads (%d) * 128", c->hidden, c->n_heads);
  if (c->hidden % 256 || c->hidden > 4096)
    return set_err(ZIMG_EUNSUPPORTED, "hidden must be a multiple of 256 and at most 4096 (got %d)", c->hidden);
  if (c->ffn <= 0 || c->ffn % 128)
    return set_err(ZIMG_EUNSUPPORTED, "ffn must be a positive multiple of 128 (got %d)", c->ffn);
  if (c->n_layers < 0 || c->n_noise_refiner < 0 || c->n_context_refiner < 0 ||
      c->n_layers + c->n_noise_refiner + c->n_context_refiner == 0)
    return set_err(ZIMG_EINVAL, "block counts must be >= 0 with at least one block");
  if (c->in_channels <= 0 || c->patch <= 0 || (c->patch * c->patch * c->in_channels) % 64)
    return set_err(ZIMG_EUNSUPPORTED, "patch*patch*in_channels must be a positive multiple of 64");
  if (c->cap_feat_dim <= 0 || c->cap_feat_dim % 256 || c->cap_feat_dim > 4096)
    return set_err(ZIMG_EUNSUPPORTED, "cap_feat_dim must be a multiple of 256 up to 4096 (got %d)", c->cap_feat_dim);
  if (c->adaln_dim <= 0 || c->adaln_dim % 256)
    return set_err(ZIMG_EUNSUPPORTED, "adaln_dim must be a positive multiple of 256 (got %d)", c->adaln_dim);
  if (c->t_mid <= 0 || c->t_mid % 256)
    return set_err(ZIMG_EUNSUPPORTED, "t_mid must be a positive multiple of 256 (got %d)", c->t_mid);
  if (c->rope_axes[0] + c->rope_axes[1] + c->rope_axes[2] != 128 || (c->rope_axes[0] | c->rope_axes[1] | c->rope_axes[2]) & 1 ||
      c->rope_axes[0] <= 0 || c->rope_axes[1] <= 0 || c->rope_axes[2] <= 0)
    return set_err(ZIMG_EUNSUPPORTED, "rope_axes must be positive, even and sum to 128");
  if (!(c->rope_theta > 0) || !std::isfinite(c->rope_theta) || !(c->t_scale > 0) || !std::isfinite(c->t_scale) ||
      !(c->max_period > 1) || !std::isfinite(c->max_period))
    return set_err(ZIMG_EINVAL, "rope_theta, t_scale must be positive and max_period > 1");
  if (!(c->norm_eps > 0) || !(c->final_eps > 0) || !std::isfinite(c->norm_eps) || !std::isfinite(c->final_eps))
    return set_err(ZIMG_EINVAL, "norm_eps and final_eps must be positive");
  if (c->max_batch < 1 || c->max_batch > 64) return set_err(ZIMG_EINVAL, "max_batch must be 1..64");
  if (c->max_image_tokens < 1 || c->max_image_tokens > (1 << 20))
    return set_err(ZIMG_EINVAL, "max_image_tokens must be 1..1048576");
  if (c->max_caption_tokens < 1 || c->max_caption_tokens > 512)
    return set_err(ZIMG_EUNSUPPORTED, "max_caption_tokens must be 1..512 (the caption limit of the model)");
  if (c->batch_invariant != 0 && c->batch_invariant != 1) return set_err(ZIMG_EINVAL, "batch_invariant must be 0 or 1");
  if (c->linear_int8 != 0 && c->linear_int8 != 1) return set_err(ZIMG_EINVAL, "linear_int8 must be 0 or 1");
  if (c->token_pad != 0 && c->token_pad != 32) return set_err(ZIMG_EUNSUPPORTED, "token_pad must be 0 or 32");
  if (c->check_finite != 0 && c->check_finite != 1) return set_err(ZIMG_EINVAL, "check_finite must be 0 or 1");
  return ZIMG_OK;
}

// ------------------------------------------------------------------ host tables

void position_ids(int L, int Hp, int Wp, int32_t* cap, int32_t* img) {
  for (int k = 0; k < L; ++k) {
    cap[3 * k] = k + 1;
    cap[3 * k + 1] = 0;
    cap[3 * k + 2] = 0;
  }
  for (int i = 0; i < Hp; ++i)
    for (int j = 0; j < Wp; ++j) {
      int32_t* r = img + 3 * (i * Wp + j);
      r[0] = L + 1;
      r[1] = i;
      r[2] = j;
    }
}

// omega per pair and the axis it belongs to
void rope_freqs(const zimg_dit_config& c, double* omega, int* axis) {
  int p = 0;
  for (int a = 0; a < 3; ++a) {
    const int d = c.rope_axes[a];
    for (int r = 0; r < d / 2; ++r, ++p) {
      omega[p] = std::pow((double)c.rope_theta, -(2.0 * r) / (double)d);
      axis[p] = a;
    }
  }
}

void rope_rows(const double* omega, const int* axis, const int32_t* ids, int64_t n, float* cs, float* sn) {
  for (int64_t s = 0; s < n; ++s)
    for (int p = 0; p < 64; ++p) {
      const double phi = (double)ids[3 * s + axis[p]] * omega[p];
      cs[s * 64 + p] = (float)std::cos(phi);
      sn[s * 64 + p] = (float)std::sin(phi);
    }
}

// ------------------------------------------------------------------ layout

// Rows of the batch: sample b's image run from img_off[b] -- its N[b] =
// Hp[b] * Wp[b] tokens, then with token padding the pad tokens up to Nseq[b]
// (a multiple of the pad size; else Nseq = N) -- padded with rows outside
// every sequence to Npad[b], a multiple of 16; all samples' image rows
// first, then each caption run (lens[b] tokens, Lseq[b] with its pad
// tokens) padded to a multiple of 16 from cap_off[b].
struct Layout {
  int B = 0;
  std::vector<int> Hl, Wl, Hp, Wp, N, Nseq, Npad, lens, Lseq, img_off, cap_off;
  int cap_base = 0, S = 0, Lsum = 0;
  bool uniform = true;  // every sample has the same latent size
};

Layout make_layout(int B, const int32_t* Hl, const int32_t* Wl, int patch, const int32_t* lens, int token_pad = 0) {
  Layout L;
  L.B = B;
  int off = 0;
  for (int b = 0; b < B; ++b) {
    L.Hl.push_back(Hl[b]);
    L.Wl.push_back(Wl[b]);
    L.Hp.push_back(Hl[b] / patch);
    L.Wp.push_back(Wl[b] / patch);
    L.N.push_back(L.Hp[b] * L.Wp[b]);
    L.Nseq.push_back(token_pad ? (int)round_up(L.N[b], token_pad) : L.N[b]);
    L.Npad.push_back((int)round_up(L.Nseq[b], 16));
    L.img_off.push_back(off);
    off += L.Npad[b];
    L.uniform = L.uniform && Hl[b] == Hl[0] && Wl[b] == Wl[0];
  }
  L.cap_base = off;
  for (int b = 0; b < B; ++b) {
    L.lens.push_back(lens[b]);
    L.Lseq.push_back(token_pad ? (int)round_up(lens[b], token_pad) : lens[b]);
    L.cap_off.push_back(off);
    off += (int)round_up(L.Lseq[b], 16);
    L.Lsum += lens[b];
  }
  L.S = off;
  return L;
}

Layout make_layout(int B, int Hl, int Wl, int patch, const int32_t* lens, int token_pad = 0) {
  std::vector<int32_t> hv(B, Hl), wv(B, Wl);
  return make_layout(B, hv.data(), wv.data(), patch, lens, token_pad);
}

// True when the B per-sample buffers of a one-size batch are consecutive
// slices of one [B, C, Hl, Wl] array.
template <class T>
bool contiguous(T* const* p, const Layout& L, int C) {
  const int64_t n = (int64_t)C * L.Hl[0] * L.Wl[0];
  for (int b = 1; b < L.B; ++b)
    if (p[b] != p[0] + b * n) return false;
  return true;
}

}  // namespace

// ------------------------------------------------------------------ engine

struct zimg_dit {
  zimg_dit_config cfg{};
  std::string err;
  int device = 0;
  hipStream_t setup = nullptr;  // the stream given at create: weight uploads, repacking, clears
  std::vector<ManifestEntry> manifest;
  std::vector<BlockSpec> blocks;
  std::vector<int> mod_index;  // per block, -1 if unmodulated
  int n_mod = 0;
  int64_t mod_stride = 0;
  bool finalized = false;

  struct BlockW {
    bf16_t *wqkv = nullptr, *wo = nullptr, *w13 = nullptr, *w2 = nullptr;
    float *an1 = nullptr, *an2 = nullptr, *fn1 = nullptr, *fn2 = nullptr, *nq = nullptr, *nk = nullptr;
    // int8 projections: codes of the same matrices (same row order) and one
    // scale per row; the bf16 copies are released once these are made
    int8_t *qqkv = nullptr, *qo = nullptr, *q13 = nullptr, *q2 = nullptr;
    float *sqkv = nullptr, *so = nullptr, *s13 = nullptr, *s2 = nullptr;
  };
  std::vector<BlockW> bw;
  bf16_t *t1w = nullptr, *t2w = nullptr, *cap_w = nullptr, *x_w = nullptr, *fin_w = nullptr, *ada_w = nullptr;
  float *t1b = nullptr, *t2b = nullptr, *capn_w = nullptr, *cap_b = nullptr, *x_b = nullptr, *fin_b = nullptr,
        *ada_b = nullptr, *pad_x = nullptr, *pad_cap = nullptr;

  // weight slots
  struct Slot {
    int kind;  // 0 bf16 matrix, 1 f32 vector, 2 w1 (interleave first), 3 w3 (interleave second)
    void* dst;
    int64_t rows, cols;
    bool set = false;
  };
  std::map<std::string, Slot> slots;

  // workspace
  int64_t S_max = 0, S_pad = 0, img_rows_max = 0, cap_rows_max = 0;
  float* x = nullptr;
  bf16_t *h = nullptr, *qkv = nullptr, *vT = nullptr, *o = nullptr, *y = nullptr, *g = nullptr, *xin = nullptr,
         *capn = nullptr;
  float *temb = nullptr, *hmid = nullptr, *cvec = nullptr, *mod = nullptr;
  // int8 projections: the block inputs h / h2 (hq), the attention output (oq)
  // and the SwiGLU product (gq) as int8 codes with one scale per row
  int8_t *hq = nullptr, *oq = nullptr, *gq = nullptr;
  float *hs = nullptr, *os = nullptr, *gs = nullptr;
  // the blocks' four norm weights, [n_blocks][4][D] (an1, an2, fn1, fn2), and
  // per forward those weights with the sample's modulation folded in,
  // [max_batch][4 n_blocks + 1][D] (the last slot: the final layer's 1 + s)
  float *normw = nullptr, *fold = nullptr;
  int32_t* mod_idx_d = nullptr;
  int64_t fold_stride = 0;
  // Per-geometry tables (RoPE cos/sin, row -> sample map, attention
  // segments and work lists) and the attention plan.  A few geometries are
  // kept on the device at once, each with its own pinned staging buffer, so
  // a caller that alternates between geometries (a guided pair and a single
  // sample, for instance) re-uploads nothing and the host never waits; a
  // slot is only rebuilt for a geometry not seen among the last kGeoSlots.
  static constexpr int kGeoSlots = 4;
  struct GeoSlot {
    std::vector<int32_t> key;  // empty: never filled
    float *cos_t = nullptr, *sin_t = nullptr;
    int32_t* row_sample = nullptr;
    zimg::AttnSeg* segs = nullptr;
    zimg::AttnItem* items = nullptr;
    void* staging = nullptr;
    hipEvent_t done = nullptr;  // the last upload from ``staging`` has completed
    uint64_t last_use = 0;
    int n_items_stage[3] = {0, 0, 0};
    int attn_full[3] = {0, 0, 0};
    int attn_split[3] = {1, 1, 1};
  } geo[kGeoSlots];
  uint64_t geo_clock = 0;
  // geometry of the previous call; when it changes, rows that were real
  // tokens may become alignment rows, which must not keep stale values
  std::vector<int32_t> last_key;
  // check_finite: the lowest stage tag whose rows held a non-finite value
  // (INT_MAX: none), and its pinned host copy
  int* finite_flag = nullptr;
  int* finite_host = nullptr;
  size_t staging_bytes = 0;
  int64_t max_items = 0;
  // views of the slot of the current geometry
  float *cos_t = nullptr, *sin_t = nullptr;
  int32_t* row_sample = nullptr;
  zimg::AttnSeg* segs = nullptr;    // [3][max_batch]
  zimg::AttnItem* items = nullptr;  // [3][max_items]
  std::vector<int32_t> table_key;
  int n_items_stage[3] = {0, 0, 0};
  int attn_full[3] = {0, 0, 0};   // (item, head) pairs of a stage computed whole
  int attn_split[3] = {1, 1, 1};  // key-range chunks of each remaining pair

  // GEMM split-K workspace (partials of the last wave's tiles); also holds
  // the partial states of split attention work
  zimg::GemmSplit split{};
  // what the GEMMs may use: nothing when results must not depend on the batch
  zimg::GemmSplit gemm_split() const { return cfg.batch_invariant ? zimg::GemmSplit{} : split; }

  // capture
  float* cap_buf = nullptr;
  size_t cap_bytes = 0;

  std::vector<void*> allocations;

  // per-kernel-class timing with HIP events on the forward's stream
  enum { K_QKV, K_OUT, K_W13, K_W2, K_ATTN, K_PRENORM, K_POSTNORM, K_EMBED, K_FINAL, K_COND, K_QUANT, K_COUNT };
  struct Prof {
    bool on = false;
    std::vector<hipEvent_t> ev;  // pairs (start, stop)
    std::vector<int> cls;
    size_t used = 0;
    int64_t count[K_COUNT] = {};
    double ms[K_COUNT] = {};
  } prof;
  int prof_harvest() {
    for (size_t i = 0; i < prof.used; ++i) {
      HIP_TRY(hipEventSynchronize(prof.ev[2 * i + 1]));
      float ms = 0.f;
      HIP_TRY(hipEventElapsedTime(&ms, prof.ev[2 * i], prof.ev[2 * i + 1]));
      prof.count[prof.cls[i]] += 1;
      prof.ms[prof.cls[i]] += ms;
    }
    prof.used = 0;
    return ZIMG_OK;
  }
  int prof_start(int c, hipStream_t s) {
    if (!prof.on) return ZIMG_OK;
    if (prof.used == prof.cls.size()) {
      int rc = prof_harvest();
      if (rc) return rc;
    }
    prof.cls[prof.used] = c;
    HIP_TRY(hipEventRecord(prof.ev[2 * prof.used], s));
    return ZIMG_OK;
  }
  int prof_stop(hipStream_t s) {
    if (!prof.on) return ZIMG_OK;
    HIP_TRY(hipEventRecord(prof.ev[2 * prof.used + 1], s));
    prof.used += 1;
    return ZIMG_OK;
  }

  int fail(int code) {
    err = g_last_error;
    return code;
  }
  template <class T>
  int dalloc(T** p, size_t count) {
    void* q = nullptr;
    const size_t bytes = count * sizeof(T);
    hipError_t e = hipMalloc(&q, bytes ? bytes : 16);
    if (e != hipSuccess)
      return set_err(e == hipErrorOutOfMemory ? ZIMG_ENOMEM : ZIMG_EHIP, "hipMalloc(%zu) failed: %s", bytes,
                     hipGetErrorString(e));
    allocations.push_back(q);
    e = hipMemsetAsync(q, 0, bytes ? bytes : 16, setup);
    if (e != hipSuccess) return set_err(ZIMG_EHIP, "hipMemsetAsync failed: %s", hipGetErrorString(e));
    *p = (T*)q;
    return ZIMG_OK;
  }

  void dfree(void* p) {
    for (size_t i = 0; i < allocations.size(); ++i)
      if (allocations[i] == p) {
        (void)hipFree(p);
        allocations.erase(allocations.begin() + i);
        return;
      }
  }

  ~zimg_dit() {
    if (finite_host) (void)hipHostFree(finite_host);
    for (hipEvent_t e : prof.ev) (void)hipEventDestroy(e);
    for (void* p : allocations) (void)hipFree(p);
    for (GeoSlot& g : geo) {
      if (g.done) (void)hipEventSynchronize(g.done);
      if (g.staging) (void)hipHostFree(g.staging);
      if (g.done) (void)hipEventDestroy(g.done);
    }
  }

  int allocate();
  int set_weight(const zimg_tensor* w);
  int finalize();
  int prepare(const Layout& L, const float* t, hipStream_t s);
  int run_block(int bi, const Layout& L, bool h_ready, int next, hipStream_t s);
  int forward(const float* const* latents, const Layout& L, const void* caps, int cap_dtype, const float* t,
              float* const* outs, hipStream_t s);
  int run_blocks(float* x_io, const Layout& L, const float* t, int first, int n, hipStream_t s);
};

int zimg_dit::allocate() {
  const zimg_dit_config& c = cfg;
  const int64_t D = c.hidden, F = c.ffn, P = (int64_t)c.patch * c.patch * c.in_channels;
  manifest = cached_manifest(c);
  blocks = block_specs(c);
  for (auto& b : blocks) mod_index.push_back(b.modulated ? n_mod++ : -1);
  mod_stride = (int64_t)n_mod * 4 * D + D;
  bw.resize(blocks.size());
  int rc;
#define ALLOC(p, n) \
  if ((rc = dalloc(&(p), (size_t)(n))) != ZIMG_OK) return rc
  const int64_t nb = (int64_t)blocks.size();
  ALLOC(normw, nb * 4 * D);
  ALLOC(mod_idx_d, nb);
  HIP_TRY(hipMemcpyAsync(mod_idx_d, mod_index.data(), nb * sizeof(int32_t), hipMemcpyHostToDevice, setup));
  HIP_TRY(hipStreamSynchronize(setup));  // mod_index is host memory
  fold_stride = (4 * nb + 1) * D;
  ALLOC(fold, (int64_t)c.max_batch * fold_stride);
  ALLOC(t1w, (int64_t)c.t_mid * c.adaln_dim);
  ALLOC(t1b, c.t_mid);
  ALLOC(t2w, (int64_t)c.adaln_dim * c.t_mid);
  ALLOC(t2b, c.adaln_dim);
  ALLOC(capn_w, c.cap_feat_dim);
  ALLOC(cap_w, D * c.cap_feat_dim);
  ALLOC(cap_b, D);
  ALLOC(x_w, D * P);
  ALLOC(x_b, D);
  ALLOC(fin_w, P * D);
  ALLOC(fin_b, P);
  ALLOC(pad_x, D);
  ALLOC(pad_cap, D);
  ALLOC(ada_w, mod_stride * c.adaln_dim);
  ALLOC(ada_b, mod_stride);
  for (size_t i = 0; i < blocks.size(); ++i) {
    BlockW& w = bw[i];
    ALLOC(w.wqkv, 3 * D * D);
    ALLOC(w.wo, D * D);
    ALLOC(w.w13, 2 * F * D);
    ALLOC(w.w2, D * F);
    w.an1 = normw + (int64_t)(4 * i + 0) * D;
    w.an2 = normw + (int64_t)(4 * i + 1) * D;
    w.fn1 = normw + (int64_t)(4 * i + 2) * D;
    w.fn2 = normw + (int64_t)(4 * i + 3) * D;
    ALLOC(w.nq, 128);
    ALLOC(w.nk, 128);
    if (c.linear_int8) {
      ALLOC(w.qqkv, 3 * D * D);
      ALLOC(w.qo, D * D);
      ALLOC(w.q13, 2 * F * D);
      ALLOC(w.q2, D * F);
      ALLOC(w.sqkv, 3 * D);
      ALLOC(w.so, D);
      ALLOC(w.s13, 2 * F);
      ALLOC(w.s2, D);
    }
  }

  // slots, named as in the manifest
  auto mat = [&](const std::string& n, void* d, int64_t r, int64_t cc, int kind = 0) {
    slots[n] = Slot{kind, d, r, cc, false};
  };
  auto vec = [&](const std::string& n, float* d, int64_t len) { slots[n] = Slot{1, d, 1, len, false}; };
  mat("t_embedder.mlp.0.weight", t1w, c.t_mid, c.adaln_dim);
  vec("t_embedder.mlp.0.bias", t1b, c.t_mid);
  mat("t_embedder.mlp.2.weight", t2w, c.adaln_dim, c.t_mid);
  vec("t_embedder.mlp.2.bias", t2b, c.adaln_dim);
  vec("cap_embedder.0.weight", capn_w, c.cap_feat_dim);
  mat("cap_embedder.1.weight", cap_w, D, c.cap_feat_dim);
  vec("cap_embedder.1.bias", cap_b, D);
  mat("all_x_embedder.2-1.weight", x_w, D, P);
  vec("all_x_embedder.2-1.bias", x_b, D);
  mat("all_final_layer.2-1.adaLN_modulation.1.weight", ada_w + (int64_t)n_mod * 4 * D * c.adaln_dim, D, c.adaln_dim);
  vec("all_final_layer.2-1.adaLN_modulation.1.bias", ada_b + (int64_t)n_mod * 4 * D, D);
  mat("all_final_layer.2-1.linear.weight", fin_w, P, D);
  vec("all_final_layer.2-1.linear.bias", fin_b, P);
  vec("x_pad_token", pad_x, D);
  vec("cap_pad_token", pad_cap, D);
  for (size_t i = 0; i < blocks.size(); ++i) {
    const std::string& p = blocks[i].prefix;
    BlockW& w = bw[i];
    mat(p + ".attention.to_q.weight", w.wqkv, D, D);
    mat(p + ".attention.to_k.weight", w.wqkv + D * D, D, D);
    mat(p + ".attention.to_v.weight", w.wqkv + 2 * D * D, D, D);
    mat(p + ".attention.to_out.0.weight", w.wo, D, D);
    vec(p + ".attention.norm_q.weight", w.nq, 128);
    vec(p + ".attention.norm_k.weight", w.nk, 128);
    mat(p + ".feed_forward.w1.weight", w.w13, F, D, 2);
    mat(p + ".feed_forward.w3.weight", w.w13, F, D, 3);
    mat(p + ".feed_forward.w2.weight", w.w2, D, F);
    vec(p + ".attention_norm1.weight", w.an1, D);
    vec(p + ".attention_norm2.weight", w.an2, D);
    vec(p + ".ffn_norm1.weight", w.fn1, D);
    vec(p + ".ffn_norm2.weight", w.fn2, D);
    if (blocks[i].modulated) {
      const int64_t k = mod_index[i];
      mat(p + ".adaLN_modulation.0.weight", ada_w + k * 4 * D * c.adaln_dim, 4 * D, c.adaln_dim);
      vec(p + ".adaLN_modulation.0.bias", ada_b + k * 4 * D, 4 * D);
    }
  }

  // workspace
  const int row_align = c.token_pad ? std::max(16, (int)c.token_pad) : 16;
  img_rows_max = (int64_t)c.max_batch * round_up(c.max_image_tokens, row_align);
  cap_rows_max = (int64_t)c.max_batch * round_up(c.max_caption_tokens, row_align);
  S_max = img_rows_max + cap_rows_max;
  S_pad = round_up(S_max, 64) + 64;
  // the attention reads a head's 128 rows of v^T through one 32-bit buffer extent
  if (S_pad > (1 << 22))
    return set_err(ZIMG_EINVAL, "max_batch x (image + caption rows) = %lld rows exceeds 2^22", (long long)S_max);
  ALLOC(x, S_max * D);
  if (c.check_finite) {
    ALLOC(finite_flag, 1);
    hipError_t e = hipHostMalloc((void**)&finite_host, sizeof(int), hipHostMallocDefault);
    if (e != hipSuccess) {
      finite_host = nullptr;
      return set_err(ZIMG_ENOMEM, "hipHostMalloc(4) failed: %s", hipGetErrorString(e));
    }
  }
  ALLOC(h, S_max * D);
  ALLOC(qkv, S_max * 3 * D);
  ALLOC(vT, (int64_t)c.n_heads * 128 * S_pad);
  ALLOC(o, S_max * D);
  ALLOC(y, S_max * D);
  ALLOC(g, S_max * F);
  if (c.linear_int8) {
    ALLOC(hq, S_max * D);
    ALLOC(oq, S_max * D);
    ALLOC(gq, S_max * F);
    ALLOC(hs, S_max);
    ALLOC(os, S_max);
    ALLOC(gs, S_max);
  }
  ALLOC(xin, img_rows_max * P);
  ALLOC(capn, cap_rows_max * c.cap_feat_dim);
  ALLOC(temb, (int64_t)c.max_batch * c.adaln_dim);
  ALLOC(hmid, (int64_t)c.max_batch * c.t_mid);
  ALLOC(cvec, (int64_t)c.max_batch * c.adaln_dim);
  ALLOC(mod, (int64_t)c.max_batch * mod_stride);
  max_items = S_max / 16 + 2 * (int64_t)c.max_batch + 8;  // q-tiles of 128 over ranges of >= 16 rows
  for (GeoSlot& gs : geo) {
    ALLOC(gs.cos_t, S_max * 64);
    ALLOC(gs.sin_t, S_max * 64);
    ALLOC(gs.row_sample, S_max);
    ALLOC(gs.segs, 3 * (int64_t)c.max_batch);
    ALLOC(gs.items, 3 * max_items);
  }
  int n_cu = 0;
  HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device));
  split.n_cu = n_cu;
  split.max_tiles = 2 * n_cu;
  split.ws_bytes = (size_t)2 * n_cu * 256 * 256 * 4;  // one partial tile per resident workgroup
  ALLOC(split.ws, split.ws_bytes / 4);
#undef ALLOC
  staging_bytes = (size_t)S_max * 64 * 4 * 2 + (size_t)S_max * 4 + 3 * c.max_batch * sizeof(zimg::AttnSeg) +
                  3 * max_items * sizeof(zimg::AttnItem);
  for (GeoSlot& gs : geo) {
    hipError_t e = hipHostMalloc(&gs.staging, staging_bytes, hipHostMallocDefault);
    if (e != hipSuccess)
      return set_err(ZIMG_ENOMEM, "hipHostMalloc(%zu) failed: %s", staging_bytes, hipGetErrorString(e));
    HIP_TRY(hipEventCreateWithFlags(&gs.done, hipEventDisableTiming));
    HIP_TRY(hipEventRecord(gs.done, setup));
  }
  HIP_TRY(hipStreamSynchronize(setup));  // the workspace clears have run
  return ZIMG_OK;
}

int zimg_dit::set_weight(const zimg_tensor* w) {
  if (!w || !w->name) return set_err(ZIMG_EINVAL, "weight tensor or its name is NULL");
  auto it = slots.find(w->name);
  if (it == slots.end()) return set_err(ZIMG_EWEIGHT, "unknown weight '%s'", w->name);
  Slot& sl = it->second;
  if (sl.set) return set_err(ZIMG_EWEIGHT, "duplicate weight '%s'", w->name);
  const ManifestEntry* me = nullptr;
  for (const auto& e : manifest)
    if (e.name == w->name) me = &e;
  if (!me || w->ndim != me->ndim) return set_err(ZIMG_EWEIGHT, "weight '%s' has rank %d, expected %d", w->name, w->ndim, me ? me->ndim : -1);
  for (int i = 0; i < me->ndim; ++i)
    if (w->shape[i] != me->shape[i])
      return set_err(ZIMG_EWEIGHT, "weight '%s' dim %d is %lld, expected %lld", w->name, i, (long long)w->shape[i],
                     (long long)me->shape[i]);
  if (!w->data) return set_err(ZIMG_EINVAL, "weight '%s' has NULL data", w->name);
  if (w->dtype != ZIMG_F32 && w->dtype != ZIMG_BF16) return set_err(ZIMG_EINVAL, "weight '%s' has unknown dtype %d", w->name, w->dtype);
  const int64_t n = sl.rows * sl.cols;
  if (sl.kind == 1) {
    std::vector<float> v(n);
    if (w->dtype == ZIMG_F32) std::memcpy(v.data(), w->data, n * 4);
    else
      for (int64_t i = 0; i < n; ++i) v[i] = bf16_to_f32(((const uint16_t*)w->data)[i]);
    HIP_TRY(hipMemcpyAsync(sl.dst, v.data(), n * 4, hipMemcpyHostToDevice, setup));
    HIP_TRY(hipStreamSynchronize(setup));  // v is released on return
  } else {
    std::vector<uint16_t> tmp;
    const uint16_t* src = (const uint16_t*)w->data;
    if (w->dtype == ZIMG_F32) {
      tmp.resize(n);
      const float* f = (const float*)w->data;
      for (int64_t i = 0; i < n; ++i) tmp[i] = f32_to_bf16(f[i]);
      src = tmp.data();
    }
    if (sl.kind == 0) {
      HIP_TRY(hipMemcpyAsync(sl.dst, src, n * 2, hipMemcpyHostToDevice, setup));
    } else {
      // interleave 32-row groups: w1 rows go to 64g + r, w3 rows to 64g + 32 + r
      const int64_t cols = sl.cols;
      const int64_t half = sl.kind == 3 ? 32 : 0;
      HIP_TRY(hipMemcpy2DAsync((bf16_t*)sl.dst + half * cols, 64 * cols * 2, src, 32 * cols * 2, 32 * cols * 2,
                               sl.rows / 32, hipMemcpyHostToDevice, setup));
    }
    HIP_TRY(hipStreamSynchronize(setup));  // the caller's array (or tmp) may go away on return
  }
  sl.set = true;
  return ZIMG_OK;
}

int zimg_dit::finalize() {
  std::string missing;
  int nmiss = 0;
  for (const auto& e : manifest)
    if (!slots[e.name].set) {
      if (nmiss < 5) missing += (missing.empty() ? "" : ", ") + e.name;
      ++nmiss;
    }
  if (nmiss) return set_err(ZIMG_EWEIGHT, "%d weight(s) missing: %s%s", nmiss, missing.c_str(), nmiss > 5 ? ", ..." : "");
  if (cfg.linear_int8) {
    // quantize every block projection per output row, then drop the bf16 copies
    const int D = cfg.hidden, F = cfg.ffn;
    for (BlockW& w : bw) {
      HIP_TRY(zimg::launch_quant_rows(w.wqkv, 1, D, w.qqkv, D, w.sqkv, 3 * D, D, 0, 1.0f, setup));
      HIP_TRY(zimg::launch_quant_rows(w.wo, 1, D, w.qo, D, w.so, D, D, 0, 1.0f, setup));
      HIP_TRY(zimg::launch_quant_rows(w.w13, 1, D, w.q13, D, w.s13, 2 * F, D, 0, 1.0f, setup));
      // w2's input is rotated by 128-point Walsh-Hadamard blocks at run time;
      // its weight rows get the same transform, and their scales the 1/128
      HIP_TRY(zimg::launch_quant_rows(w.w2, 1, F, w.q2, F, w.s2, D, F, 1, 1.0f / 128.0f, setup));
    }
    HIP_TRY(hipStreamSynchronize(setup));
    for (BlockW& w : bw) {
      for (bf16_t** m : {&w.wqkv, &w.wo, &w.w13, &w.w2}) {
        dfree(*m);
        *m = nullptr;
      }
    }
  }
  finalized = true;
  return ZIMG_OK;
}

// Build (or reuse) the RoPE tables, row->sample map and attention work lists
// for this geometry, then compute the timestep conditioning and every
// block's modulation.
int zimg_dit::prepare(const Layout& L, const float* t, hipStream_t s) {
  const zimg_dit_config& c = cfg;
  std::vector<int32_t> key = {L.B};
  for (int b = 0; b < L.B; ++b) {
    key.push_back(L.Hl[b]);
    key.push_back(L.Wl[b]);
    key.push_back(L.lens[b]);
  }
  int slot = -1;
  for (int i = 0; i < kGeoSlots; ++i)
    if (geo[i].key == key) slot = i;
  if (slot < 0) {
    // a new geometry: rebuild the least recently used slot
    slot = 0;
    for (int i = 1; i < kGeoSlots; ++i)
      if (geo[i].last_use < geo[slot].last_use) slot = i;
    GeoSlot& G = geo[slot];
    G.key.clear();
    // its staging buffer was last read by an upload at least one geometry
    // change ago; that upload has normally long completed
    HIP_TRY(hipEventSynchronize(G.done));
    int* n_items_stage = G.n_items_stage;
    int* attn_full = G.attn_full;
    int* attn_split = G.attn_split;
    char* st = (char*)G.staging;
    float* cs = (float*)st;
    float* sn = cs + L.S * 64;
    int32_t* rs = (int32_t*)(sn + L.S * 64);
    zimg::AttnSeg* sg = (zimg::AttnSeg*)(rs + L.S);
    zimg::AttnItem* itm = (zimg::AttnItem*)(sg + 3 * c.max_batch);
    for (int64_t i = 0; i < (int64_t)L.S * 64; ++i) {
      cs[i] = 1.0f;
      sn[i] = 0.0f;
    }
    for (int i = 0; i < L.S; ++i) rs[i] = 0;
    double omega[64];
    int axis[64];
    rope_freqs(c, omega, axis);
    std::vector<int32_t> cap_ids, img_ids;
    for (int b = 0; b < L.B; ++b) {
      // positions of the caption run (with its pad tokens, which continue it)
      // and of the image tokens after it; image pad tokens keep the
      // identity rows (position 0) the tables were cleared to
      cap_ids.assign((size_t)L.Lseq[b] * 3, 0);
      img_ids.assign((size_t)L.N[b] * 3, 0);
      position_ids(L.Lseq[b], L.Hp[b], L.Wp[b], cap_ids.data(), img_ids.data());
      rope_rows(omega, axis, img_ids.data(), L.N[b], cs + (int64_t)L.img_off[b] * 64, sn + (int64_t)L.img_off[b] * 64);
      rope_rows(omega, axis, cap_ids.data(), L.Lseq[b], cs + (int64_t)L.cap_off[b] * 64, sn + (int64_t)L.cap_off[b] * 64);
      for (int i = 0; i < L.Npad[b]; ++i) rs[L.img_off[b] + i] = b;
      for (int i = 0; i < (int)round_up(L.Lseq[b], 16); ++i) rs[L.cap_off[b] + i] = b;
    }
    // segments and q-tiles of 128 rows per stage
    for (int stg = 0; stg < 3; ++stg) {
      int ni = 0;
      for (int b = 0; b < L.B; ++b) {
        zimg::AttnSeg& q = sg[stg * c.max_batch + b];
        q = zimg::AttnSeg{{0, 0}, {0, 0}};
        int k = 0;
        if (stg != 1) {
          q.r0[k] = L.img_off[b];
          q.n[k++] = L.Nseq[b];
        }
        if (stg != 0) {
          q.r0[k] = L.cap_off[b];
          q.n[k++] = L.Lseq[b];
        }
        for (int r = 0; r < k; ++r)
          for (int q0 = 0; q0 < q.n[r]; q0 += 128) {
            if (ni >= max_items) return set_err(ZIMG_EINVAL, "internal: attention work list overflow");
            itm[stg * max_items + ni++] = zimg::AttnItem{q.r0[r] + q0, std::min(128, q.n[r] - q0), b, 0};
          }
      }
      n_items_stage[stg] = ni;
      // Two attention workgroups are resident per CU.  When the pairs of the
      // last, partial round would fill at most half of those slots, each of
      // them is split into chunks of its key tiles (at least two tiles per
      // chunk) so that the round is filled, with one merge launch after.
      const int P = 2 * split.n_cu, total = ni * c.n_heads, r = total % P;
      attn_full[stg] = total;
      attn_split[stg] = 1;
      if (!c.batch_invariant && r > 0 && 2 * r <= P) {
        int tmin = 1 << 30;
        for (int lid = total - r; lid < total; ++lid) {
          const zimg::AttnSeg& q = sg[stg * c.max_batch + itm[stg * max_items + lid % ni].seg];
          tmin = std::min(tmin, (q.n[0] + 63) / 64 + (q.n[1] + 63) / 64);
        }
        const int sp = std::min(std::min(P / r, tmin / 2), 16);
        if (sp >= 2 && (size_t)r * sp * zimg::ATTN_PART_FLOATS * 4 <= split.ws_bytes) {
          attn_full[stg] = total - r;
          attn_split[stg] = sp;
        }
      }
    }
    HIP_TRY(hipMemcpyAsync(G.cos_t, cs, (size_t)L.S * 64 * 4, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(G.sin_t, sn, (size_t)L.S * 64 * 4, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(G.row_sample, rs, (size_t)L.S * 4, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(G.segs, sg, 3 * c.max_batch * sizeof(zimg::AttnSeg), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(G.items, itm, 3 * max_items * sizeof(zimg::AttnItem), hipMemcpyHostToDevice, s));
    HIP_TRY(hipEventRecord(G.done, s));
    G.key = key;
  }
  if (key != last_key) {
    // Alignment rows (in no attention segment) are computed like tokens from
    // rows of xin, capn and o that no call writes, so they stay finite as
    // long as those rows start finite; after a change of geometry they may
    // hold an earlier call's tokens, which are cleared here.  Attention reads
    // the alignment rows just past a range's end as keys of weight 0, and
    // 0 * v must not become NaN.
    HIP_TRY(zimg::launch_fill(reinterpret_cast<float*>(xin), 0.0f, img_rows_max * (c.patch * c.patch * c.in_channels) / 2, s));
    HIP_TRY(zimg::launch_fill(reinterpret_cast<float*>(capn), 0.0f, cap_rows_max * c.cap_feat_dim / 2, s));
    HIP_TRY(zimg::launch_fill(reinterpret_cast<float*>(o), 0.0f, S_max * c.hidden / 2, s));
    last_key = key;
  }
  {
    GeoSlot& G = geo[slot];
    G.last_use = ++geo_clock;
    cos_t = G.cos_t;
    sin_t = G.sin_t;
    row_sample = G.row_sample;
    segs = G.segs;
    items = G.items;
    for (int i = 0; i < 3; ++i) {
      n_items_stage[i] = G.n_items_stage[i];
      attn_full[i] = G.attn_full[i];
      attn_split[i] = G.attn_split[i];
    }
    table_key = key;
  }

  // timestep embedding -> MLP -> every modulation vector
  zimg::TimeArgs ta{};
  for (int b = 0; b < L.B; ++b) ta.t[b] = t[b];
  const int64_t D = c.hidden;
  int rc = prof_start(K_COND, s);
  if (rc) return rc;
  HIP_TRY(zimg::launch_timestep_embed(ta, L.B, c.adaln_dim, c.t_scale, c.max_period, temb, s));
  HIP_TRY(zimg::launch_gemv(t1w, t1b, temb, c.adaln_dim, hmid, c.t_mid, c.t_mid, c.adaln_dim, L.B, 0, s));
  HIP_TRY(zimg::launch_gemv(t2w, t2b, hmid, c.t_mid, cvec, c.adaln_dim, c.adaln_dim, c.t_mid, L.B, 1, s));
  if (n_mod)
    HIP_TRY(zimg::launch_gemv(ada_w, ada_b, cvec, c.adaln_dim, mod, mod_stride, (int)(n_mod * 4 * D), c.adaln_dim,
                              L.B, 0, s));
  HIP_TRY(zimg::launch_gemv(ada_w + n_mod * 4 * D * c.adaln_dim, ada_b + n_mod * 4 * D, cvec, c.adaln_dim,
                            mod + n_mod * 4 * D, mod_stride, (int)D, c.adaln_dim, L.B, 1, s));
  HIP_TRY(zimg::launch_fold_mod(mod, mod_stride, normw, mod_idx_d, (int)blocks.size(), n_mod, (int)D, L.B, fold, s));
  return prof_stop(s);
}

static void stage_rows(const Layout& L, int stage, int& r0, int& r1) {
  r0 = stage == 1 ? L.cap_base : 0;
  r1 = stage == 0 ? L.cap_base : L.S;
}

// One block on rows of its stage.  ``h_ready``: h already holds this block's
// modulated pre-norm (fused into the previous block's last kernel).
// ``next``: 0 no fused follow-up, 1 the next block's pre-norm (same rows),
// 2 the final layer's LayerNorm on the image rows.
int zimg_dit::run_block(int bi, const Layout& L, bool h_ready, int next, hipStream_t s) {
  const zimg_dit_config& c = cfg;
  const int D = c.hidden, F = c.ffn, H = c.n_heads;
  const BlockW& w = bw[bi];
  const int stage = blocks[bi].stage;
  int r0, r1;
  stage_rows(L, stage, r0, r1);
  const int M = r1 - r0;
  // folded norm weights of this block: 0 attention pre, 1 attention post,
  // 2 FFN pre, 3 FFN post
  auto mref = [&](int chunk) { return zimg::VecRef{fold + (int64_t)(4 * bi + chunk) * D, fold_stride}; };
  const bool i8 = c.linear_int8 != 0;
  if (!h_ready) {
    zimg::PreNormArgs pa{x, mref(0), row_sample, h, r0, r1, D, c.norm_eps, 0, hq, hs};
    PROFILED(K_PRENORM, zimg::launch_pre_norm(pa, s));
  }
  // operands of a projection: bf16, or int8 codes with per-row scales
  zimg::GemmArgs ga{};
  auto operands = [&](const bf16_t* a16, const int8_t* a8, const float* sa, const bf16_t* w16, const int8_t* w8,
                      const float* sw, int64_t ld) {
    ga.i8 = i8;
    ga.A = i8 ? (const void*)(a8 + (int64_t)r0 * ld) : (const void*)(a16 + (int64_t)r0 * ld);
    ga.W = i8 ? (const void*)w8 : (const void*)w16;
    ga.lda = ga.ldw = ld;
    ga.ep.sa = i8 ? sa + r0 : nullptr;
    ga.ep.sw = i8 ? sw : nullptr;
  };
  operands(h, hq, hs, w.wqkv, w.qqkv, w.sqkv, D);
  ga.M = M;
  ga.N = 3 * D;
  ga.K = D;
  // epilogue: QK-RMSNorm + RoPE in place, V transposed into vT
  ga.epi = zimg::EPI_QKV_ROPE;
  ga.ep.C = qkv + (int64_t)r0 * 3 * D;
  ga.ep.ldc = 3 * D;
  ga.ep.wq = w.nq;
  ga.ep.wk = w.nk;
  ga.ep.cos_t = cos_t;
  ga.ep.sin_t = sin_t;
  ga.ep.vT = vT;
  ga.ep.trow0 = r0;
  ga.ep.S_pad = (int)S_pad;
  ga.ep.D = D;
  ga.ep.eps = c.norm_eps;
  ga.role = zimg::ROLE_QKV;
  ga.split = gemm_split();
  PROFILED(K_QKV, zimg::launch_gemm(ga, s));
  ga.ep = zimg::EpiArgs{};
  ga.epi = zimg::EPI_BF16;

  zimg::AttnArgs aa{qkv,
                    vT,
                    o,
                    items + stage * max_items,
                    segs + stage * c.max_batch,
                    n_items_stage[stage],
                    H,
                    (int)S_pad,
                    (int)S_max,
                    (float)(1.4426950408889634 / std::sqrt(128.0)),
                    attn_full[stage],
                    attn_split[stage],
                    split.ws};
  PROFILED(K_ATTN, zimg::launch_attention(aa, s));

  if (i8) PROFILED(K_QUANT, zimg::launch_quant_rows(o + (int64_t)r0 * D, 1, D, oq + (int64_t)r0 * D, D, os + r0, M, D, 0, 1.0f, s));
  operands(o, oq, os, w.wo, w.qo, w.so, D);
  ga.N = D;
  ga.ep.C = y + (int64_t)r0 * D;
  ga.ep.ldc = D;
  ga.role = zimg::ROLE_OUT;
  ga.split = gemm_split();
  PROFILED(K_OUT, zimg::launch_gemm(ga, s));

  zimg::PostNormArgs pn{};
  pn.x = x;
  pn.y = y;
  pn.wg = mref(1);
  pn.r0 = r0;
  pn.r1 = r1;
  pn.n0 = r0;
  pn.n1 = r1;
  pn.wn = mref(2);
  pn.next_kind = 0;
  pn.next_eps = c.norm_eps;
  pn.row_sample = row_sample;
  pn.h = h;
  pn.D = D;
  pn.eps = c.norm_eps;
  pn.hq = hq;
  pn.hs = hs;
  PROFILED(K_POSTNORM, zimg::launch_post_norm(pn, s));

  operands(h, hq, hs, w.w13, w.q13, w.s13, D);
  ga.N = 2 * F;
  ga.epi = zimg::EPI_SWIGLU;
  ga.ep.C = g + (int64_t)r0 * F;
  ga.ep.ldc = F;
  ga.role = zimg::ROLE_W13;
  ga.split = gemm_split();
  PROFILED(K_W13, zimg::launch_gemm(ga, s));

  if (i8) PROFILED(K_QUANT, zimg::launch_quant_rows(g + (int64_t)r0 * F, 1, F, gq + (int64_t)r0 * F, F, gs + r0, M, F, 1, 1.0f, s));
  operands(g, gq, gs, w.w2, w.q2, w.s2, F);
  ga.N = D;
  ga.K = F;
  ga.epi = zimg::EPI_BF16;
  ga.ep.C = y + (int64_t)r0 * D;
  ga.ep.ldc = D;
  ga.role = zimg::ROLE_W2;
  ga.split = gemm_split();
  PROFILED(K_W2, zimg::launch_gemm(ga, s));

  pn.wg = mref(3);
  if (next == 1) {
    pn.wn = zimg::VecRef{fold + (int64_t)(4 * (bi + 1)) * D, fold_stride};
    pn.next_kind = 0;
    pn.next_eps = c.norm_eps;
  } else if (next == 2) {
    pn.n0 = 0;
    pn.n1 = L.cap_base;
    pn.wn = zimg::VecRef{fold + (int64_t)(4 * blocks.size()) * D, fold_stride};
    pn.next_kind = 1;
    pn.next_eps = c.final_eps;
    pn.hq = nullptr;  // the final layer takes bf16
    pn.hs = nullptr;
  } else {
    pn.n0 = pn.n1 = 0;
  }
  PROFILED(K_POSTNORM, zimg::launch_post_norm(pn, s));
  return ZIMG_OK;
}

int zimg_dit::forward(const float* const* latents, const Layout& L, const void* caps, int cap_dtype, const float* t,
                      float* const* outs, hipStream_t s) {
  const zimg_dit_config& c = cfg;
  const int D = c.hidden, P = c.patch * c.patch * c.in_channels;
  int rc = prepare(L, t, s);
  if (rc) return rc;
  // patch embed -> image rows of x (fp32, bias); caption embed -> caption rows.
  // A batch of one latent size (contiguous latents) is patchified in one
  // launch; otherwise sample by sample.
  rc = prof_start(K_EMBED, s);
  if (rc) return rc;
  if (L.uniform && contiguous(latents, L, c.in_channels))
    HIP_TRY(zimg::launch_patchify(latents[0], xin, L.B, c.in_channels, L.Hp[0], L.Wp[0], c.patch, L.Npad[0], s));
  else
    for (int b = 0; b < L.B; ++b)
      HIP_TRY(zimg::launch_patchify(latents[b], xin + (int64_t)L.img_off[b] * P, 1, c.in_channels, L.Hp[b], L.Wp[b],
                                    c.patch, L.Npad[b], s));
  zimg::GemmArgs ga{};
  ga.A = xin;
  ga.lda = P;
  ga.W = x_w;
  ga.ldw = P;
  ga.M = L.cap_base;
  ga.N = D;
  ga.K = P;
  ga.epi = zimg::EPI_F32_BIAS;
  ga.role = zimg::ROLE_EMBED;
  ga.split = gemm_split();
  ga.ep.C = x;
  ga.ep.ldc = D;
  ga.ep.bias = x_b;
  HIP_TRY(zimg::launch_gemm(ga, s));
  int64_t src = 0;
  for (int b = 0; b < L.B; ++b) {
    const void* cb = cap_dtype == ZIMG_BF16 ? (const void*)((const uint16_t*)caps + src * c.cap_feat_dim)
                                            : (const void*)((const float*)caps + src * c.cap_feat_dim);
    HIP_TRY(zimg::launch_rows_rmsnorm(cb, cap_dtype == ZIMG_BF16, capn_w,
                                      capn + (int64_t)(L.cap_off[b] - L.cap_base) * c.cap_feat_dim, L.lens[b],
                                      c.cap_feat_dim, c.norm_eps, s));
    src += L.lens[b];
  }
  ga.A = capn;
  ga.lda = c.cap_feat_dim;
  ga.W = cap_w;
  ga.ldw = c.cap_feat_dim;
  ga.M = L.S - L.cap_base;
  ga.K = c.cap_feat_dim;
  ga.ep.C = x + (int64_t)L.cap_base * D;
  ga.ep.bias = cap_b;
  HIP_TRY(zimg::launch_gemm(ga, s));
  // pad tokens: the learned embeddings replace whatever the embed GEMMs left
  // in those rows
  for (int b = 0; b < L.B; ++b) {
    HIP_TRY(zimg::launch_set_rows(x, D, pad_x, L.img_off[b] + L.N[b], L.Nseq[b] - L.N[b], s));
    HIP_TRY(zimg::launch_set_rows(x, D, pad_cap, L.cap_off[b] + L.lens[b], L.Lseq[b] - L.lens[b], s));
  }
  rc = prof_stop(s);
  if (rc) return rc;
  // check_finite: every stage's sequence rows (each sample's image and
  // caption runs; alignment rows are never read) are scanned after it runs
  auto scan_rows = [&](int tag) -> hipError_t {
    for (int b = 0; b < L.B; ++b) {
      hipError_t e = zimg::launch_scan_finite(x + (int64_t)L.img_off[b] * D, (int64_t)L.Nseq[b] * D, tag, finite_flag, s);
      if (e == hipSuccess)
        e = zimg::launch_scan_finite(x + (int64_t)L.cap_off[b] * D, (int64_t)L.Lseq[b] * D, tag, finite_flag, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  if (c.check_finite) {
    HIP_TRY(zimg::launch_set_int(finite_flag, INT_MAX, s));
    HIP_TRY(scan_rows(0));
  }
  const size_t slot_bytes = (size_t)L.S * D * 4;
  if (cap_buf) HIP_TRY(hipMemcpyAsync(cap_buf, x, slot_bytes, hipMemcpyDeviceToDevice, s));

  const int nb = (int)blocks.size();
  bool h_ready = false;
  bool final_ready = false;
  for (int bi = 0; bi < nb; ++bi) {
    int next = 0;
    if (bi + 1 < nb && blocks[bi + 1].stage == blocks[bi].stage) next = 1;
    else if (bi + 1 == nb && blocks[bi].stage != 1) next = 2;  // image rows are inside the block's rows
    rc = run_block(bi, L, h_ready, next, s);
    if (rc) return rc;
    h_ready = next == 1;
    final_ready = next == 2;
    if (cap_buf) HIP_TRY(hipMemcpyAsync((char*)cap_buf + (size_t)(bi + 1) * slot_bytes, x, slot_bytes,
                                        hipMemcpyDeviceToDevice, s));
    if (c.check_finite) HIP_TRY(scan_rows(bi + 1));
  }
  rc = prof_start(K_FINAL, s);
  if (rc) return rc;
  if (!final_ready) {
    zimg::PreNormArgs pa{x, zimg::VecRef{fold + (int64_t)(4 * blocks.size()) * D, fold_stride}, row_sample, h, 0,
                         L.cap_base, D, c.final_eps, 1};
    HIP_TRY(zimg::launch_pre_norm(pa, s));
  }
  // final linear + unpatchify: one launch for a batch of one latent size
  // (contiguous outputs), else one per sample
  auto final_gemm = [&](int r0, int rows, int b0, float* dst) -> hipError_t {
    zimg::GemmArgs gf{};
    gf.A = h + (int64_t)r0 * D;
    gf.lda = D;
    gf.W = fin_w;
    gf.ldw = D;
    gf.M = rows;
    gf.N = P;
    gf.K = D;
    gf.epi = zimg::EPI_UNPATCH;
    gf.role = zimg::ROLE_FINAL;
    gf.split = gemm_split();
    gf.ep.C = dst;
    gf.ep.bias = fin_b;
    gf.ep.ntok = L.N[b0];
    gf.ep.npad = L.Npad[b0];
    gf.ep.Hp = L.Hp[b0];
    gf.ep.Wp = L.Wp[b0];
    gf.ep.C_ch = c.in_channels;
    gf.ep.patch = c.patch;
    return zimg::launch_gemm(gf, s);
  };
  if (L.uniform && contiguous(outs, L, c.in_channels)) {
    HIP_TRY(final_gemm(0, L.cap_base, 0, outs[0]));
  } else {
    for (int b = 0; b < L.B; ++b) HIP_TRY(final_gemm(L.img_off[b], L.Npad[b], b, outs[b]));
  }
  rc = prof_stop(s);
  if (rc || !c.check_finite) return rc;
  // check_finite: scan the outputs, then wait for the result
  const int nb_all = (int)blocks.size();
  for (int b = 0; b < L.B; ++b)
    HIP_TRY(zimg::launch_scan_finite(outs[b], (int64_t)c.in_channels * L.Hp[b] * c.patch * L.Wp[b] * c.patch, nb_all + 1,
                                     finite_flag, s));
  HIP_TRY(hipMemcpyAsync(finite_host, finite_flag, sizeof(int), hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  const int bad = *finite_host;
  if (bad == INT_MAX) return ZIMG_OK;
  if (bad == 0) return set_err(ZIMG_ENONFINITE, "non-finite values in the sequence after the embeddings");
  if (bad <= nb_all)
    return set_err(ZIMG_ENONFINITE, "non-finite values in the sequence after block %d (%s)", bad - 1,
                   blocks[bad - 1].prefix.c_str());
  return set_err(ZIMG_ENONFINITE, "non-finite values in the model output");
}

int zimg_dit::run_blocks(float* x_io, const Layout& L, const float* t, int first, int n, hipStream_t s) {
  int rc = prepare(L, t, s);
  if (rc) return rc;
  const size_t bytes = (size_t)L.S * cfg.hidden * 4;
  HIP_TRY(hipMemcpyAsync(x, x_io, bytes, hipMemcpyDeviceToDevice, s));
  bool h_ready = false;
  for (int bi = first; bi < first + n; ++bi) {
    const int next = (bi + 1 < first + n && blocks[bi + 1].stage == blocks[bi].stage) ? 1 : 0;
    rc = run_block(bi, L, h_ready, next, s);
    if (rc) return rc;
    h_ready = next == 1;
  }
  HIP_TRY(hipMemcpyAsync(x_io, x, bytes, hipMemcpyDeviceToDevice, s));
  return ZIMG_OK;
}

// ------------------------------------------------------------------ C ABI

namespace {

int validate_inputs(const zimg_dit* h, int32_t B, const int32_t* Hl, const int32_t* Wl, const int32_t* lens,
                    const float* t) {
  const zimg_dit_config& c = h->cfg;
  if (!h->finalized) return set_err(ZIMG_ESTATE, "weights not finalized (missing zimg_dit_finalize?)");
  if (B < 1 || B > c.max_batch) return set_err(ZIMG_EINVAL, "batch %d out of range 1..%d", B, c.max_batch);
  if (!Hl || !Wl) return set_err(ZIMG_EINVAL, "latent sizes must be host arrays, got NULL");
  for (int b = 0; b < B; ++b) {
    if (Hl[b] <= 0 || Wl[b] <= 0 || Hl[b] % c.patch || Wl[b] % c.patch)
      return set_err(ZIMG_EINVAL,
                     "latent %dx%d: sides must be positive multiples of the patch size %d (image sides multiples of 16)",
                     Hl[b], Wl[b], c.patch);
    const int64_t ntok = (int64_t)(Hl[b] / c.patch) * (Wl[b] / c.patch);
    if (ntok > c.max_image_tokens)
      return set_err(ZIMG_EINVAL, "%lld image tokens exceed max_image_tokens %d", (long long)ntok, c.max_image_tokens);
  }
  if (!lens || !t) return set_err(ZIMG_EINVAL, "caption_lens and t must be host arrays, got NULL");
  for (int b = 0; b < B; ++b) {
    if (lens[b] < 1 || lens[b] > c.max_caption_tokens)
      return set_err(ZIMG_EINVAL, "caption %d has length %d, outside 1..%d", b, lens[b], c.max_caption_tokens);
    if (!std::isfinite(t[b])) return set_err(ZIMG_EINVAL, "t[%d] is not finite", b);
  }
  return ZIMG_OK;
}

int validate_inputs(const zimg_dit* h, int32_t B, int32_t Hl, int32_t Wl, const int32_t* lens, const float* t) {
  if (B < 1 || B > 4096) return set_err(ZIMG_EINVAL, "batch %d out of range 1..%d", B, h->cfg.max_batch);
  std::vector<int32_t> hv(B, Hl), wv(B, Wl);
  return validate_inputs(h, B, hv.data(), wv.data(), lens, t);
}

// Forward on per-sample latent / output buffers (validated arguments).
int run_forward(zimg_dit* h, const float* const* latents, int32_t B, const int32_t* Hl, const int32_t* Wl,
                const void* caption_feats, int32_t cap_dtype, const int32_t* caption_lens, const float* t,
                float* const* outs, void* stream) {
  if (!caption_feats) return set_err(ZIMG_EINVAL, "caption_feats must be non-NULL");
  for (int b = 0; b < B; ++b)
    if (!latents[b] || !outs[b]) return set_err(ZIMG_EINVAL, "latent and output buffers must be non-NULL");
  if (cap_dtype != ZIMG_F32 && cap_dtype != ZIMG_BF16) return set_err(ZIMG_EINVAL, "cap_dtype must be ZIMG_F32 or ZIMG_BF16");
  Layout L = make_layout(B, Hl, Wl, h->cfg.patch, caption_lens, h->cfg.token_pad);
  if (h->cap_buf) {
    const size_t need = (size_t)(h->blocks.size() + 1) * L.S * h->cfg.hidden * 4;
    if (h->cap_bytes < need) return set_err(ZIMG_EINVAL, "capture buffer has %zu bytes, needs %zu", h->cap_bytes, need);
  }
  return h->forward(latents, L, caption_feats, cap_dtype, t, outs, (hipStream_t)stream);
}

}  // namespace

// ------------------------------------------------------------------ attention op

namespace {

// Work list and split plan of the attention op for B samples with segments
// seg [B][4] = (r0 of the first range, its rows, r0 of the second, its rows).
struct AttnOpPlan {
  int n_items = 0, n_full = 0, split = 1;
  int rows = 0;           // rows of qkv the segments reach (the key rows' bound)
  size_t header = 0;      // bytes of the work list at the start of the workspace
  size_t part_bytes = 0;  // bytes of split partials the plan uses
  zimg::AttnPlanArgs pa{};
};

int attention_op_plan(int32_t H, int32_t B, const int32_t* seg, int64_t S_pad, size_t ws_bytes, AttnOpPlan& P) {
  if (H < 1 || H > 256) return set_err(ZIMG_EINVAL, "attention: H %d outside 1..256", H);
  if (B < 1 || B > zimg::ATTN_OP_MAX_B) return set_err(ZIMG_EINVAL, "attention: B %d outside 1..%d", B, zimg::ATTN_OP_MAX_B);
  if (!seg) return set_err(ZIMG_EINVAL, "attention: segments array is NULL");
  if (S_pad < 64 || S_pad % 8 || S_pad > (1 << 22)) return set_err(ZIMG_EINVAL, "attention: S_pad %lld must be a multiple of 8 in 64..2^22", (long long)S_pad);
  P.pa.B = B;
  int n = 0;
  for (int b = 0; b < B; ++b) {
    zimg::AttnSeg& q = P.pa.seg[b];
    for (int r = 0; r < 2; ++r) {
      const int64_t r0 = seg[4 * b + 2 * r], len = seg[4 * b + 2 * r + 1];
      if (len < 0 || r0 < 0 || r0 % 8) return set_err(ZIMG_EINVAL, "attention: sample %d range %d: start %lld must be a non-negative multiple of 8 and length %lld non-negative", b, r, (long long)r0, (long long)len);
      if (r == 0 && len < 1) return set_err(ZIMG_EINVAL, "attention: sample %d: the first range is empty", b);
      if (len > 0 && r0 + (len + 63) / 64 * 64 > S_pad)
        return set_err(ZIMG_EINVAL, "attention: sample %d range %d: rows %lld..%lld (rounded up to 64 keys) exceed S_pad %lld", b, r, (long long)r0, (long long)(r0 + len), (long long)S_pad);
      q.r0[r] = (int)r0;
      q.n[r] = (int)len;
      if (len > 0) P.rows = std::max(P.rows, (int)(r0 + len));
    }
    P.pa.item_off[b] = n;
    n += (q.n[0] + 127) / 128 + (q.n[1] + 127) / 128;
  }
  P.pa.item_off[B] = n;
  P.n_items = n;
  P.header = (1024 + (size_t)16 * n + 255) / 256 * 256;
  if ((int64_t)n * H > (1 << 30)) return set_err(ZIMG_EINVAL, "attention: too many work items");
  if (ws_bytes < P.header)
    return set_err(ZIMG_EINVAL, "attention: workspace of %zu bytes is smaller than the %zu-byte work list", ws_bytes, P.header);
  int dev = 0, n_cu = 0;
  HIP_TRY(hipGetDevice(&dev));
  HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  // the engine's rule: two attention workgroups are resident per CU; a last
  // round at most half full is split along keys (chunks of >= 2 key tiles)
  const int total = n * H, Pslots = 2 * n_cu, r = total % Pslots;
  P.n_full = total;
  P.split = 1;
  if (r > 0 && 2 * r <= Pslots) {
    int tmin = 1 << 30;
    for (int lid = total - r; lid < total; ++lid) {
      const int item = lid % n;
      int b = 0;
      while (P.pa.item_off[b + 1] <= item) ++b;
      const zimg::AttnSeg& q = P.pa.seg[b];
      tmin = std::min(tmin, (q.n[0] + 63) / 64 + (q.n[1] + 63) / 64);
    }
    int sp = std::min(std::min(Pslots / r, tmin / 2), 16);
    while (sp >= 2 && P.header + (size_t)r * sp * zimg::ATTN_PART_FLOATS * 4 > ws_bytes) --sp;
    if (sp >= 2) {
      P.n_full = total - r;
      P.split = sp;
      P.part_bytes = (size_t)r * sp * zimg::ATTN_PART_FLOATS * 4;
    }
  }
  return ZIMG_OK;
}

int attention_op(const void* qkv, const void* vT, int64_t S_pad, void* out, int32_t H, int32_t B, const int32_t* seg,
                 void* ws, size_t ws_bytes, hipStream_t s) {
  if (!qkv || !vT || !out || !ws) return set_err(ZIMG_EINVAL, "attention: NULL buffer");
  if (((uintptr_t)qkv & 15) || ((uintptr_t)vT & 15) || ((uintptr_t)out & 7) || ((uintptr_t)ws & 255))
    return set_err(ZIMG_EINVAL, "attention: qkv and vT must be 16-byte, out 8-byte and the workspace 256-byte aligned");
  AttnOpPlan P;
  int rc = attention_op_plan(H, B, seg, S_pad, ws_bytes, P);
  if (rc) return rc;
  char* w = (char*)ws;
  P.pa.segs = (zimg::AttnSeg*)w;
  P.pa.items = (zimg::AttnItem*)(w + 1024);
  HIP_TRY(zimg::launch_attention_plan(P.pa, s));
  zimg::AttnArgs aa{(const bf16_t*)qkv,
                    (const bf16_t*)vT,
                    (bf16_t*)out,
                    P.pa.items,
                    P.pa.segs,
                    P.n_items,
                    H,
                    (int)S_pad,
                    P.rows,
                    (float)(1.4426950408889634 / std::sqrt(128.0)),
                    P.n_full,
                    P.split,
                    (float*)(w + P.header)};
  HIP_TRY(zimg::launch_attention(aa, s));
  return ZIMG_OK;
}

}  // namespace

namespace zimg {
const zimg_dit_config* handle_config(const zimg_dit* h) { return h ? &h->cfg : nullptr; }
bool handle_finalized(const zimg_dit* h) { return h && h->finalized; }
}  // namespace zimg

extern "C" {

const char* zimg_last_error(void) { return g_last_error.c_str(); }

void zimg_dit_default_config(zimg_dit_config* c) {
  if (!c) return;
  *c = zimg_dit_config{};
  c->hidden = 3840;
  c->n_heads = 30;
  c->ffn = 10240;
  c->n_layers = 30;
  c->n_noise_refiner = 2;
  c->n_context_refiner = 2;
  c->in_channels = 16;
  c->patch = 2;
  c->cap_feat_dim = 2560;
  c->adaln_dim = 256;
  c->t_mid = 1024;
  c->rope_axes[0] = 32;
  c->rope_axes[1] = 48;
  c->rope_axes[2] = 48;
  c->rope_theta = 256.0f;
  c->t_scale = 1000.0f;
  c->max_period = 10000.0f;
  c->norm_eps = 1e-5f;
  c->final_eps = 1e-6f;
  c->max_batch = 1;
  c->max_image_tokens = 4096;
  c->token_pad = 0;
  c->max_caption_tokens = 512;
}

int zimg_dit_check_config(const zimg_dit_config* cfg) {
  g_last_error.clear();
  return check_config(cfg);
}

int zimg_dit_manifest_size(const zimg_dit_config* cfg, int32_t* n) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!n) return set_err(ZIMG_EINVAL, "n_tensors is NULL");
  *n = (int32_t)cached_manifest(*cfg).size();
  return ZIMG_OK;
}

int zimg_dit_manifest_entry(const zimg_dit_config* cfg, int32_t index, const char** name, int32_t* ndim,
                            int64_t shape[4]) {
  int rc = check_config(cfg);
  if (rc) return rc;
  const auto& m = cached_manifest(*cfg);
  if (index < 0 || index >= (int32_t)m.size()) return set_err(ZIMG_EINVAL, "manifest index %d out of range", index);
  if (name) *name = m[index].name.c_str();
  if (ndim) *ndim = m[index].ndim;
  if (shape)
    for (int i = 0; i < 4; ++i) shape[i] = m[index].shape[i];
  return ZIMG_OK;
}

int zimg_dit_alloc(const zimg_dit_config* cfg, void* stream, zimg_dit** out) {
  g_last_error.clear();
  if (!out) return set_err(ZIMG_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev < 1)
    return set_err(ZIMG_EHIP, "no HIP device available: %s", e != hipSuccess ? hipGetErrorString(e) : "0 devices");
  std::unique_ptr<zimg_dit> h(new zimg_dit());
  h->cfg = *cfg;
  h->setup = (hipStream_t)stream;
  HIP_TRY(hipGetDevice(&h->device));
  rc = h->allocate();
  if (rc) return rc;
  *out = h.release();
  return ZIMG_OK;
}

int zimg_dit_set_weight(zimg_dit* h, const zimg_tensor* w) {
  if (!h) return set_err(ZIMG_EINVAL, "handle is NULL");
  if (h->finalized) return h->fail(set_err(ZIMG_ESTATE, "weights already finalized"));
  int rc = h->set_weight(w);
  return rc ? h->fail(rc) : ZIMG_OK;
}

int zimg_dit_finalize(zimg_dit* h) {
  if (!h) return set_err(ZIMG_EINVAL, "handle is NULL");
  int rc = h->finalize();
  return rc ? h->fail(rc) : ZIMG_OK;
}

int zimg_dit_create(const zimg_dit_config* cfg, const zimg_tensor* weights, int32_t n_weights, void* stream,
                    zimg_dit** out) {
  if (!out) return set_err(ZIMG_EINVAL, "out is NULL");
  *out = nullptr;
  if (n_weights < 0 || (n_weights > 0 && !weights)) return set_err(ZIMG_EINVAL, "bad weights array");
  zimg_dit* h = nullptr;
  int rc = zimg_dit_alloc(cfg, stream, &h);
  if (rc) return rc;
  for (int32_t i = 0; i < n_weights && !rc; ++i) rc = zimg_dit_set_weight(h, &weights[i]);
  if (!rc) rc = zimg_dit_finalize(h);
  if (rc) {
    delete h;
    return rc;
  }
  *out = h;
  return ZIMG_OK;
}

void zimg_dit_destroy(zimg_dit* h) { delete h; }

const char* zimg_dit_last_error(const zimg_dit* h) { return h ? h->err.c_str() : "handle is NULL"; }

int zimg_dit_set_capture(zimg_dit* h, float* dev_buf, size_t bytes) {
  if (!h) return set_err(ZIMG_EINVAL, "handle is NULL");
  h->cap_buf = dev_buf;
  h->cap_bytes = dev_buf ? bytes : 0;
  return ZIMG_OK;
}

int zimg_dit_forward(zimg_dit* h, const float* latent, int32_t B, int32_t Hl, int32_t Wl, const void* caption_feats,
                     int32_t cap_dtype, const int32_t* caption_lens, const float* t, float* out, void* stream) {
  g_last_error.clear();
  if (!h) return set_err(ZIMG_EINVAL, "handle is NULL");
  int rc = validate_inputs(h, B, Hl, Wl, caption_lens, t);
  if (rc) return h->fail(rc);
  if (!latent || !out) return h->fail(set_err(ZIMG_EINVAL, "latent, caption_feats and out must be non-NULL"));
  const int64_t n = (int64_t)h->cfg.in_channels * Hl * Wl;
  std::vector<const float*> lat(B);
  std::vector<float*> outs(B);
  std::vector<int32_t> hv(B, Hl), wv(B, Wl);
  for (int b = 0; b < B; ++b) {
    lat[b] = latent + b * n;
    outs[b] = out + b * n;
  }
  rc = run_forward(h, lat.data(), B, hv.data(), wv.data(), caption_feats, cap_dtype, caption_lens, t, outs.data(), stream);
  return rc ? h->fail(rc) : ZIMG_OK;
}

int zimg_dit_forward_varsize(zimg_dit* h, const float* const* latents, int32_t B, const int32_t* Hl, const int32_t* Wl,
                             const void* caption_feats, int32_t cap_dtype, const int32_t* caption_lens, const float* t,
                             float* const* outs, void* stream) {
  g_last_error.clear();
  if (!h) return set_err(ZIMG_EINVAL, "handle is NULL");
  if (!latents || !outs) return h->fail(set_err(ZIMG_EINVAL, "latents and outs must be host arrays, got NULL"));
  int rc = validate_inputs(h, B, Hl, Wl, caption_lens, t);
  if (rc) return h->fail(rc);
  rc = run_forward(h, latents, B, Hl, Wl, caption_feats, cap_dtype, caption_lens, t, outs, stream);
  return rc ? h->fail(rc) : ZIMG_OK;
}

int zimg_dit_run_blocks(zimg_dit* h, float* x_io, int32_t B, int32_t Hl, int32_t Wl, const int32_t* caption_lens,
                        const float* t, int32_t first_block, int32_t n_blocks, void* stream) {
  g_last_error.clear();
  if (!h) return set_err(ZIMG_EINVAL, "handle is NULL");
  int rc = validate_inputs(h, B, Hl, Wl, caption_lens, t);
  if (rc) return h->fail(rc);
  if (!x_io) return h->fail(set_err(ZIMG_EINVAL, "x_io is NULL"));
  if (first_block < 0 || n_blocks < 1 || first_block + n_blocks > (int32_t)h->blocks.size())
    return h->fail(set_err(ZIMG_EINVAL, "blocks [%d, %d) out of range 0..%zu", first_block, first_block + n_blocks,
                           h->blocks.size()));
  Layout L = make_layout(B, Hl, Wl, h->cfg.patch, caption_lens, h->cfg.token_pad);
  rc = h->run_blocks(x_io, L, t, first_block, n_blocks, (hipStream_t)stream);
  return rc ? h->fail(rc) : ZIMG_OK;
}

int zimg_row_layout_varsize(int32_t B, const int32_t* n_image_tokens, const int32_t* caption_lens, int32_t* img_off,
                            int32_t* cap_off, int32_t* S_total) {
  g_last_error.clear();
  if (B < 1 || !n_image_tokens || !caption_lens) return set_err(ZIMG_EINVAL, "bad layout arguments");
  for (int b = 0; b < B; ++b)
    if (caption_lens[b] < 1 || n_image_tokens[b] < 1) return set_err(ZIMG_EINVAL, "token counts must be >= 1");
  int64_t off = 0;
  for (int b = 0; b < B; ++b) {
    if (img_off) img_off[b] = (int32_t)off;
    off += round_up(n_image_tokens[b], 16);
  }
  for (int b = 0; b < B; ++b) {
    if (cap_off) cap_off[b] = (int32_t)off;
    off += round_up(caption_lens[b], 16);
  }
  if (S_total) *S_total = (int32_t)off;
  return ZIMG_OK;
}

int zimg_row_layout(int32_t B, int32_t n_image_tokens, const int32_t* caption_lens, int32_t* img_off, int32_t* cap_off,
                    int32_t* S_total) {
  if (B < 1) return set_err(ZIMG_EINVAL, "bad layout arguments");
  std::vector<int32_t> n(B, n_image_tokens);
  return zimg_row_layout_varsize(B, n.data(), caption_lens, img_off, cap_off, S_total);
}

int zimg_position_ids(int32_t L, int32_t Hp, int32_t Wp, int32_t* cap_ids, int32_t* img_ids) {
  g_last_error.clear();
  if (L < 0 || Hp < 0 || Wp < 0 || (L && !cap_ids) || (Hp * Wp && !img_ids))
    return set_err(ZIMG_EINVAL, "bad position-id arguments");
  std::vector<int32_t> dummy(3);
  position_ids(L, Hp, Wp, L ? cap_ids : dummy.data(), Hp * Wp ? img_ids : dummy.data());
  return ZIMG_OK;
}

int zimg_rope_tables(const zimg_dit_config* cfg, const int32_t* ids, int64_t S, float* cs, float* sn) {
  g_last_error.clear();
  int rc = check_config(cfg);
  if (rc) return rc;
  if (S < 0 || (S && (!ids || !cs || !sn))) return set_err(ZIMG_EINVAL, "bad rope-table arguments");
  double omega[64];
  int axis[64];
  rope_freqs(*cfg, omega, axis);
  rope_rows(omega, axis, ids, S, cs, sn);
  return ZIMG_OK;
}

int zimg_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int32_t M, int32_t N,
                   int32_t K, int32_t epilogue, const float* bias, void* stream) {
  g_last_error.clear();
  zimg::GemmArgs g{};
  g.A = (const bf16_t*)A;
  g.lda = lda;
  g.W = (const bf16_t*)W;
  g.ldw = ldw;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi = epilogue;
  g.ep.C = C;
  g.ep.ldc = ldc;
  g.ep.bias = bias;
  g.role = zimg::ROLE_ANY;
  if (epilogue == zimg::EPI_UNPATCH || epilogue == zimg::EPI_QKV_ROPE)
    return set_err(ZIMG_EUNSUPPORTED, "epilogue %d is internal", epilogue);
  if (const char* m = zimg::gemm_check(g)) return set_err(ZIMG_EINVAL, "%s", m);
  const int64_t need = epilogue == zimg::EPI_SWIGLU ? N / 2 : N;
  if (ldc < need) return set_err(ZIMG_EINVAL, "ldc %lld smaller than the output width %lld", (long long)ldc, (long long)need);
  HIP_TRY(zimg::launch_gemm(g, (hipStream_t)stream));
  return ZIMG_OK;
}

int zimg_gemm_i8(const void* A, int64_t lda, const float* sa, const void* W, int64_t ldw, const float* sw, void* C,
                 int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue, const float* bias, void* stream) {
  g_last_error.clear();
  zimg::GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.W = W;
  g.ldw = ldw;
  g.M = M;
  g.N = N;
  g.K = K;
  g.i8 = 1;
  g.epi = epilogue;
  g.ep.C = C;
  g.ep.ldc = ldc;
  g.ep.bias = bias;
  g.ep.sa = sa;
  g.ep.sw = sw;
  g.role = zimg::ROLE_ANY;
  if (epilogue == zimg::EPI_UNPATCH || epilogue == zimg::EPI_QKV_ROPE)
    return set_err(ZIMG_EUNSUPPORTED, "epilogue %d is internal", epilogue);
  if (const char* m = zimg::gemm_check(g)) return set_err(ZIMG_EINVAL, "%s", m);
  const int64_t need = epilogue == zimg::EPI_SWIGLU ? N / 2 : N;
  if (ldc < need) return set_err(ZIMG_EINVAL, "ldc %lld smaller than the output width %lld", (long long)ldc, (long long)need);
  HIP_TRY(zimg::launch_gemm(g, (hipStream_t)stream));
  return ZIMG_OK;
}

int zimg_quantize_rows(const void* x, int32_t x_dtype, int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                       int32_t rows, int32_t K, int32_t rotate_block, void* stream) {
  g_last_error.clear();
  if (rows < 0 || K <= 0 || K % 8 || K > 16384) return set_err(ZIMG_EINVAL, "need rows >= 0 and K a multiple of 8 in 8..16384");
  if (x_dtype != ZIMG_F32 && x_dtype != ZIMG_BF16) return set_err(ZIMG_EINVAL, "unknown dtype %d", x_dtype);
  if (ldx < K || ldq < K || ldx % 8 || ldq % 8) return set_err(ZIMG_EINVAL, "ldx, ldq must be multiples of 8 and >= K");
  if (rows > 0 && (!x || !q || !scale)) return set_err(ZIMG_EINVAL, "NULL buffer");
  const uintptr_t xa = (uintptr_t)x, qa = (uintptr_t)q;
  if (rows > 0 && ((xa & 15) || (qa & 7))) return set_err(ZIMG_EINVAL, "x must be 16-byte and q 8-byte aligned");
  if (rotate_block != 0 && rotate_block != 128) return set_err(ZIMG_EINVAL, "rotate_block must be 0 or 128");
  if (rotate_block && K % 128) return set_err(ZIMG_EINVAL, "rotation needs K a multiple of 128");
  HIP_TRY(zimg::launch_quant_rows(x, x_dtype == ZIMG_BF16, ldx, q, ldq, scale, rows, K, rotate_block != 0, 1.0f,
                                  (hipStream_t)stream));
  return ZIMG_OK;
}

int zimg_dit_profile(zimg_dit* h, int32_t enable) {
  g_last_error.clear();
  if (!h) return set_err(ZIMG_EINVAL, "handle is NULL");
  if (enable) {
    if (h->prof.ev.empty()) {
      const size_t pairs = 4096;
      h->prof.ev.resize(2 * pairs, nullptr);
      h->prof.cls.resize(pairs, 0);
      for (auto& e : h->prof.ev) {
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return h->fail(set_err(ZIMG_EHIP, "hipEventCreate failed: %s", hipGetErrorString(err)));
      }
    }
    h->prof.used = 0;
    for (int i = 0; i < zimg_dit::K_COUNT; ++i) {
      h->prof.count[i] = 0;
      h->prof.ms[i] = 0.0;
    }
  }
  h->prof.on = enable != 0;
  return ZIMG_OK;
}

int zimg_dit_profile_read(zimg_dit* h, zimg_kernel_stat* stats, int32_t max_stats, int32_t* n_stats) {
  static const char* names[zimg_dit::K_COUNT] = {"gemm_qkv", "gemm_out", "gemm_w13_swiglu", "gemm_w2", "attention",
                                                 "pre_norm", "post_norm", "embed", "final_layer",
                                                 "conditioning", "quant"};
  g_last_error.clear();
  if (!h) return set_err(ZIMG_EINVAL, "handle is NULL");
  if (max_stats < 0 || (max_stats > 0 && !stats)) return set_err(ZIMG_EINVAL, "bad stats array");
  int rc = h->prof_harvest();
  if (rc) return h->fail(rc);
  for (int i = 0; i < zimg_dit::K_COUNT && i < max_stats; ++i) {
    stats[i].name = names[i];
    stats[i].launches = h->prof.count[i];
    stats[i].total_ms = h->prof.ms[i];
  }
  if (n_stats) *n_stats = zimg_dit::K_COUNT;
  return ZIMG_OK;
}

int zimg_cfg_euler_step(float* x, const float* out_cond, const float* out_uncond, float guidance, float dt,
                        int64_t n, void* stream) {
  g_last_error.clear();
  if (n < 0) return set_err(ZIMG_EINVAL, "n is negative");
  if (n > 0 && (!x || !out_cond || !out_uncond)) return set_err(ZIMG_EINVAL, "NULL buffer");
  if (!std::isfinite(dt) || !std::isfinite(guidance)) return set_err(ZIMG_EINVAL, "dt or guidance is not finite");
  if (n > 0 && (x == out_cond || x == out_uncond)) return set_err(ZIMG_EINVAL, "x aliases a model output");
  HIP_TRY(zimg::launch_cfg_euler(x, out_cond, out_uncond, guidance, dt, n, (hipStream_t)stream));
  return ZIMG_OK;
}

int zimg_dit_attention_plan(zimg_dit* h, int32_t stage, int32_t out[3]) {
  g_last_error.clear();
  if (!h || !out) return set_err(ZIMG_EINVAL, "NULL argument");
  if (stage < 0 || stage > 2) return set_err(ZIMG_EINVAL, "stage %d is not 0, 1 or 2", stage);
  if (h->table_key.empty()) return set_err(ZIMG_ESTATE, "no forward has set a geometry yet");
  out[0] = h->n_items_stage[stage] * h->cfg.n_heads;
  out[1] = h->attn_full[stage];
  out[2] = h->attn_split[stage];
  return ZIMG_OK;
}


int zimg_attention_workspace_size(int32_t H, int32_t B, const int32_t* seg, int64_t S_pad, size_t* bytes) {
  if (!bytes) return set_err(ZIMG_EINVAL, "bytes is NULL");
  AttnOpPlan P;
  int rc = attention_op_plan(H, B, seg, S_pad, (size_t)-1, P);
  if (rc) return rc;
  *bytes = P.header + P.part_bytes;
  return ZIMG_OK;
}

int zimg_attention(const void* qkv, const void* vT, int64_t S_pad, void* out, int32_t H, int32_t B,
                   const int32_t* seg, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  return attention_op(qkv, vT, S_pad, out, H, B, seg, workspace, ws_bytes, (hipStream_t)stream);
}

// The same op with the library's static device scratch in place of a
// workspace: nothing is allocated.  The scratch address of the current
// device is looked up on its first use there (hipGetSymbolAddress, with that
// device current) and kept.
int zimg_attention_noalloc(const void* qkv, const void* vT, int64_t S_pad, void* out, int32_t H, int32_t B,
                           const int32_t* seg, void* stream) {
  g_last_error.clear();
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipError_t e = hipSuccess;
  void* ws = zimg::attention_scratch(dev, &e);
  if (!ws) return set_err(ZIMG_EHIP, "attention: device scratch of device %d unavailable: %s", dev, hipGetErrorString(e));
  AttnOpPlan P;
  int rc = attention_op_plan(H, B, seg, S_pad, zimg::ATTN_SCRATCH_BYTES, P);
  if (rc) return set_err(rc, "attention (no-allocation entry point, %zu-byte scratch): %s", zimg::ATTN_SCRATCH_BYTES,
                         g_last_error.c_str());
  return attention_op(qkv, vT, S_pad, out, H, B, seg, ws, zimg::ATTN_SCRATCH_BYTES, (hipStream_t)stream);
}

// The flow-match schedule, in float64 and in the order of operations of the
// definition: base sigmas as an evenly spaced ramp from 1 down to 1/N
// (sigma_i = 1 + i * ((1/N - 1) / (N - 1)), the last one exactly 1/N), the
// shift s * sigma / (1 + (s - 1) * sigma), a final 0, and the model times
// (1000 - 1000 sigma') / 1000.  Contraction into fused multiply-adds is off,
// so every product and sum is rounded on its own.
#pragma clang fp contract(off)
int zimg_flowmatch_schedule(int32_t n_steps, double shift, double* sigmas, double* t) {
  if (n_steps < 1 || n_steps > (1 << 20)) return set_err(ZIMG_EINVAL, "n_steps %d outside 1..2^20", n_steps);
  if (!std::isfinite(shift) || shift <= 0.0) return set_err(ZIMG_EINVAL, "shift must be finite and positive");
  if (!sigmas || !t) return set_err(ZIMG_EINVAL, "output array is NULL");
  const double start = 1.0, stop = 1.0 / n_steps;
  const double step = n_steps > 1 ? (stop - start) / (double)(n_steps - 1) : 0.0;
  for (int32_t i = 0; i < n_steps; ++i) {
    double base = (double)i * step;
    base = base + start;
    if (i == n_steps - 1) base = stop;
    const double num = shift * base;
    const double den = 1.0 + (shift - 1.0) * base;
    const double sp = num / den;
    sigmas[i] = sp;
    const double thousand_sp = 1000.0 * sp;
    t[i] = (1000.0 - thousand_sp) / 1000.0;
  }
  sigmas[n_steps] = 0.0;
  return ZIMG_OK;
}
#pragma clang fp contract(on)

int zimg_euler_step(float* x, const float* model_out, float dt, int64_t n, void* stream) {
  g_last_error.clear();
  if (!x || !model_out || n < 0) return set_err(ZIMG_EINVAL, "bad Euler-step arguments");
  if (!std::isfinite(dt)) return set_err(ZIMG_EINVAL, "dt is not finite");
  HIP_TRY(zimg::launch_euler(x, model_out, dt, n, (hipStream_t)stream));
  return ZIMG_OK;
}

}  // extern "C"
