// Host orchestrator and C ABI: weight validation / packing, workspace planning, the per-forward
// launch sequence, and the per-stage entry points.
//
// Forward sequence (diffusers WanTransformer3DModel.forward and WanTransformerBlock.forward as printed
// on the WanPipeline notes page; block order from the Wan2.1 walk-through page, section 5.2):
//   patchify -> patch-embed GEMM (fp32 residual x) ; sinusoid -> time MLP (fp32) ; text projection
//   per block: [x += gate2 * ffn of the previous block] LN1+mod -> QKV GEMM -> QK RMSNorm + RoPE
//              -> V transpose -> attention -> O GEMM
//              [x += gate1 * attn] LN2 affine -> Q2 GEMM -> RMSNorm ; ctx K/V GEMM -> RMSNorm(k)
//              -> V transpose -> cross attention -> O2 GEMM
//              [x += cross-attn] LN3+mod -> FFN1 GEMM (GELU) -> FFN2 GEMM
//   head: [x += gate2 * ffn] LN + (table + temb) modulation -> proj_out GEMM -> unpatchify
// Each residual add [..] runs inside the LayerNorm kernel that follows it: the branch's last Linear
// writes bf16 (as the branch outputs are in the bf16 model), and x stays fp32.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <string>
#include <unordered_map>
#include <vector>

#include "common.h"
#include "launch.h"
#include "wan_dit.h"
#include "wan_ops.h"

namespace {

thread_local std::string g_err;

wan_status fail(wan_status st, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr, what)                                                                \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(WAN_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
  } while (0)

struct BlockW {
  bf16_t *wqkv, *wo, *wq2, *wkv2, *wo2, *w1, *w2;
  float *bqkv, *bo, *bq2, *bkv2, *bo2, *b1, *b2;
  float *gq, *gk, *gq2, *gk2, *n2w, *n2b, *table;
  bf16_t* wkvi;   // image branch: [add_k_proj; add_v_proj] [2D, D]
  float *bkvi, *gki;
};

// Bump allocator over one device allocation (256-byte aligned slices).
struct Arena {
  char* base = nullptr;
  size_t size = 0, used = 0;
  template <typename T>
  T* take(int64_t count) {
    size_t bytes = ((size_t)count * sizeof(T) + 255) & ~(size_t)255;
    T* p = (T*)(base ? base + used : nullptr);
    used += bytes;
    return p;
  }
};

}  // namespace

struct wan_dit {
  wan_dit_config cfg;
  int device = 0;
  void* wmem = nullptr;
  void* wsmem = nullptr;
  size_t wbytes = 0, wsbytes = 0;
  int64_t kp_pe = 0, n_out = 0;
  // packed weights
  bf16_t* w_pe; float* b_pe;
  float *t_w1, *t_b1, *t_w2, *t_b2, *t_wp, *t_bp;
  bf16_t *c_w1, *c_w2; float *c_b1, *c_b2;
  bf16_t *i_w1, *i_w2; float *i_b1, *i_b2;   // image MLP (max_image_len > 0)
  int64_t kp_img = 0;
  std::vector<BlockW> blocks;
  float* head_table; bf16_t* w_out; float* b_out;
  // workspace
  bf16_t *P, *y, *qkv, *vt, *attn, *br, *hbuf, *text_bf, *ctx_h, *ctx, *kv2, *vt2;
  bf16_t *img_bf, *img_h, *img_ctx, *kvi, *vti;   // image branch
  float *x, *z, *t_s, *t_h, *temb, *tproj, *rope, *t_dup;
  float* attn_ws;   // key-split partials of the attention's last round and its redo flags
  int64_t attn_ws_bytes = 0;
  float* gemm_ws;   // stream-K partial tiles of the GEMMs' last round
  int64_t gemm_ws_bytes = 0;
  int64_t ldv_max, ldv2_max, ldvi_max, rows_max, trows_max;
  // opt-in timing of the self-attention launches (wan_dit_time_attention): event pairs, start then end
  std::vector<hipEvent_t> att_ev;
  int64_t att_used = 0;
};

namespace {

int64_t numel(const int64_t* shape, int ndim) {
  int64_t n = 1;
  for (int i = 0; i < ndim; ++i) n *= shape[i];
  return n;
}

std::string shape_str(const int64_t* shape, int ndim) {
  std::string s = "[";
  for (int i = 0; i < ndim; ++i) {
    if (i) s += ",";
    s += std::to_string(shape[i]);
  }
  return s + "]";
}

wan_status check_config(const wan_dit_config* c) {
  if (!c) return fail(WAN_ERR_INVALID_ARG, "config is NULL");
  if (c->head_dim != 128) return fail(WAN_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", c->head_dim);
  if (c->num_heads <= 0 || c->dim != c->num_heads * c->head_dim)
    return fail(WAN_ERR_INVALID_ARG, "dim (%d) must equal num_heads (%d) * head_dim", c->dim, c->num_heads);
  if (c->dim % 512 != 0 || c->dim > 12288)
    return fail(WAN_ERR_UNSUPPORTED, "dim must be a multiple of 512 and <= 12288 (got %d)", c->dim);
  if (c->dim > 6144) return fail(WAN_ERR_UNSUPPORTED, "dim above 6144 not supported by the LayerNorm kernel");
  if (c->ffn_dim <= 0 || c->ffn_dim % 64 != 0) return fail(WAN_ERR_UNSUPPORTED, "ffn_dim must be a positive multiple of 64");
  if (c->num_layers < 0) return fail(WAN_ERR_INVALID_ARG, "num_layers < 0");
  if (c->in_channels <= 0 || c->out_channels <= 0) return fail(WAN_ERR_INVALID_ARG, "channel counts must be positive");
  if (c->text_dim <= 0 || c->text_dim % 64 != 0) return fail(WAN_ERR_UNSUPPORTED, "text_dim must be a positive multiple of 64");
  if (c->freq_dim <= 0 || c->freq_dim % 2 != 0) return fail(WAN_ERR_UNSUPPORTED, "freq_dim must be positive and even");
  if (c->patch_t != 1 || c->patch_h != 2 || c->patch_w != 2)
    return fail(WAN_ERR_UNSUPPORTED, "only the (1,2,2) patch is implemented");
  if (c->rope_dim_t <= 0 || c->rope_dim_h <= 0 || c->rope_dim_w <= 0 || (c->rope_dim_t | c->rope_dim_h | c->rope_dim_w) & 1 ||
      c->rope_dim_t + c->rope_dim_h + c->rope_dim_w != c->head_dim)
    return fail(WAN_ERR_INVALID_ARG, "rope dims must be positive, even and sum to head_dim");
  if (!(c->eps > 0.f)) return fail(WAN_ERR_INVALID_ARG, "eps must be positive");
  if (!(c->rope_theta > 1.0)) return fail(WAN_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (c->max_batch <= 0 || c->max_tokens <= 0 || c->max_text_len <= 0)
    return fail(WAN_ERR_INVALID_ARG, "max_batch, max_tokens and max_text_len must be positive");
  if (c->max_image_len < 0) return fail(WAN_ERR_INVALID_ARG, "max_image_len must be >= 0");
  if (c->max_image_len > 0 && (c->image_dim <= 0 || c->image_dim % 8 != 0))
    return fail(WAN_ERR_UNSUPPORTED, "image_dim must be a positive multiple of 8 (got %d)", c->image_dim);
  return WAN_OK;
}

struct Expect {
  std::string name;
  std::vector<int64_t> shape;
};

std::vector<Expect> expected_weights(const wan_dit_config& c) {
  const int64_t D = c.dim, Fd = c.ffn_dim;
  std::vector<Expect> e;
  auto lin = [&](const std::string& n, int64_t o, int64_t i) {
    e.push_back({n + ".weight", {o, i}});
    e.push_back({n + ".bias", {o}});
  };
  e.push_back({"patch_embedding.weight", {D, c.in_channels, c.patch_t, c.patch_h, c.patch_w}});
  e.push_back({"patch_embedding.bias", {D}});
  lin("time_embedder.linear_1", D, c.freq_dim);
  lin("time_embedder.linear_2", D, D);
  lin("time_proj", 6 * D, D);
  lin("text_embedder.linear_1", D, c.text_dim);
  lin("text_embedder.linear_2", D, D);
  if (c.max_image_len > 0) {
    lin("image_embedder.linear_1", D, c.image_dim);
    lin("image_embedder.linear_2", D, D);
  }
  for (int k = 0; k < c.num_layers; ++k) {
    const std::string p = "blocks." + std::to_string(k) + ".";
    e.push_back({p + "scale_shift_table", {1, 6, D}});
    for (const char* a : {"attn1", "attn2"}) {
      for (const char* pr : {"to_q", "to_k", "to_v", "to_out"}) lin(p + a + "." + pr, D, D);
      e.push_back({p + a + ".norm_q.weight", {D}});
      e.push_back({p + a + ".norm_k.weight", {D}});
    }
    if (c.max_image_len > 0) {
      lin(p + "attn2.add_k_proj", D, D);
      lin(p + "attn2.add_v_proj", D, D);
      e.push_back({p + "attn2.norm_added_k.weight", {D}});
    }
    e.push_back({p + "norm2.weight", {D}});
    e.push_back({p + "norm2.bias", {D}});
    lin(p + "ffn.proj_in", Fd, D);
    lin(p + "ffn.proj_out", D, Fd);
  }
  e.push_back({"scale_shift_table", {1, 2, D}});
  lin("proj_out", 4LL * c.out_channels, D);
  return e;
}

// Plan (or, with a live base pointer, carve) the packed-weight arena.
void plan_weights(wan_dit* h, Arena& ar) {
  const wan_dit_config& c = h->cfg;
  const int64_t D = c.dim, Fd = c.ffn_dim;
  h->w_pe = ar.take<bf16_t>(D * h->kp_pe);
  h->b_pe = ar.take<float>(D);
  h->t_w1 = ar.take<float>(D * c.freq_dim); h->t_b1 = ar.take<float>(D);
  h->t_w2 = ar.take<float>(D * D); h->t_b2 = ar.take<float>(D);
  h->t_wp = ar.take<float>(6 * D * D); h->t_bp = ar.take<float>(6 * D);
  h->c_w1 = ar.take<bf16_t>(D * c.text_dim); h->c_b1 = ar.take<float>(D);
  h->c_w2 = ar.take<bf16_t>(D * D); h->c_b2 = ar.take<float>(D);
  const bool img = c.max_image_len > 0;
  h->i_w1 = img ? ar.take<bf16_t>(D * h->kp_img) : nullptr; h->i_b1 = img ? ar.take<float>(D) : nullptr;
  h->i_w2 = img ? ar.take<bf16_t>(D * D) : nullptr; h->i_b2 = img ? ar.take<float>(D) : nullptr;
  h->blocks.resize(c.num_layers);
  for (auto& b : h->blocks) {
    b.wqkv = ar.take<bf16_t>(3 * D * D); b.bqkv = ar.take<float>(3 * D);
    b.wo = ar.take<bf16_t>(D * D); b.bo = ar.take<float>(D);
    b.wq2 = ar.take<bf16_t>(D * D); b.bq2 = ar.take<float>(D);
    b.wkv2 = ar.take<bf16_t>(2 * D * D); b.bkv2 = ar.take<float>(2 * D);
    b.wo2 = ar.take<bf16_t>(D * D); b.bo2 = ar.take<float>(D);
    b.w1 = ar.take<bf16_t>(Fd * D); b.b1 = ar.take<float>(Fd);
    b.w2 = ar.take<bf16_t>(D * Fd); b.b2 = ar.take<float>(D);
    b.gq = ar.take<float>(D); b.gk = ar.take<float>(D); b.gq2 = ar.take<float>(D); b.gk2 = ar.take<float>(D);
    b.n2w = ar.take<float>(D); b.n2b = ar.take<float>(D);
    b.table = ar.take<float>(6 * D);
    b.wkvi = img ? ar.take<bf16_t>(2 * D * D) : nullptr;
    b.bkvi = img ? ar.take<float>(2 * D) : nullptr;
    b.gki = img ? ar.take<float>(D) : nullptr;
  }
  h->head_table = ar.take<float>(2 * D);
  h->w_out = ar.take<bf16_t>(h->n_out * D);
  h->b_out = ar.take<float>(h->n_out);
}

void plan_workspace(wan_dit* h, Arena& ar) {
  const wan_dit_config& c = h->cfg;
  const int64_t D = c.dim, Fd = c.ffn_dim;
  const int64_t Mx = c.max_batch * c.max_tokens;
  const int64_t R = c.per_token_timestep ? Mx : c.max_batch;
  const int64_t Tx = c.max_batch * c.max_text_len;
  h->rows_max = Mx;
  h->trows_max = R;
  h->ldv_max = round_up(c.max_tokens, 64);
  h->ldv2_max = round_up(c.max_text_len, 64);
  h->P = ar.take<bf16_t>(Mx * h->kp_pe);
  h->x = ar.take<float>(Mx * D);
  h->y = ar.take<bf16_t>(Mx * D);
  h->qkv = ar.take<bf16_t>(Mx * 3 * D);
  h->vt = ar.take<bf16_t>(c.max_batch * D * h->ldv_max);
  h->attn = ar.take<bf16_t>(Mx * D);
  h->br = ar.take<bf16_t>(Mx * D);
  h->hbuf = ar.take<bf16_t>(Mx * Fd);
  h->z = ar.take<float>(Mx * h->n_out);
  h->t_s = ar.take<float>(R * c.freq_dim);
  h->t_h = ar.take<float>(R * D);
  h->temb = ar.take<float>(R * D);
  h->tproj = ar.take<float>(R * 6 * D);
  h->rope = ar.take<float>(rope_table_floats(1024, 1024, 1024, c.rope_dim_t, c.rope_dim_h, c.rope_dim_w));
  h->text_bf = ar.take<bf16_t>(Tx * c.text_dim);
  h->ctx_h = ar.take<bf16_t>(Tx * D);
  h->ctx = ar.take<bf16_t>(Tx * D);
  h->kv2 = ar.take<bf16_t>(Tx * 2 * D);
  h->vt2 = ar.take<bf16_t>(c.max_batch * D * h->ldv2_max);
  const int64_t Ix = c.max_batch * c.max_image_len;
  h->ldvi_max = round_up(c.max_image_len, 64);
  h->img_bf = ar.take<bf16_t>(Ix * h->kp_img);
  h->img_h = ar.take<bf16_t>(Ix * D);
  h->img_ctx = ar.take<bf16_t>(Ix * D);
  h->kvi = ar.take<bf16_t>(Ix * 2 * D);
  h->vti = ar.take<bf16_t>(c.max_image_len ? c.max_batch * D * h->ldvi_max : 0);
  h->t_dup = ar.take<float>(c.max_batch * (c.per_token_timestep ? c.max_tokens : 1));
  h->attn_ws_bytes = attention_workspace_bytes(c.max_batch, c.max_tokens, c.num_heads);
  h->attn_ws = ar.take<float>(h->attn_ws_bytes / 4);
  h->gemm_ws_bytes = gemm_workspace_bytes();
  h->gemm_ws = ar.take<float>(h->gemm_ws_bytes / 4);
}

void release_events(wan_dit* h) {
  for (hipEvent_t e : h->att_ev) (void)hipEventDestroy(e);
  h->att_ev.clear();
  h->att_used = 0;
}

void free_handle(wan_dit* h) {
  if (!h) return;
  release_events(h);
  if (h->wmem) (void)hipFree(h->wmem);
  if (h->wsmem) (void)hipFree(h->wsmem);
  delete h;
}

wan_status check_tensor(const wan_tensor* t, const char* what) {
  if (!t) return fail(WAN_ERR_INVALID_ARG, "%s is NULL", what);
  if (t->ndim < 1 || t->ndim > 6) return fail(WAN_ERR_SHAPE, "%s: ndim %d out of range", what, t->ndim);
  if (t->dtype != WAN_F32 && t->dtype != WAN_BF16) return fail(WAN_ERR_DTYPE, "%s: unknown dtype %d", what, t->dtype);
  for (int i = 0; i < t->ndim; ++i)
    if (t->shape[i] < 0) return fail(WAN_ERR_SHAPE, "%s: negative dimension", what);
  if (!t->data && numel(t->shape, t->ndim) > 0) return fail(WAN_ERR_INVALID_ARG, "%s: data is NULL", what);
  return WAN_OK;
}

}  // namespace

// =====================================================================================================
// C ABI
// =====================================================================================================

extern "C" const char* wan_dit_last_error(void) { return g_err.c_str(); }

extern "C" int64_t wan_dit_device_bytes(const wan_dit* h) { return h ? (int64_t)(h->wbytes + h->wsbytes) : 0; }

extern "C" void wan_dit_destroy(wan_dit* h) { free_handle(h); }

extern "C" wan_status wan_dit_time_attention(wan_dit* h, int64_t max_launches) {
  g_err.clear();
  if (!h) return fail(WAN_ERR_INVALID_ARG, "handle is NULL");
  if (max_launches < 0 || max_launches > (int64_t)1 << 20)
    return fail(WAN_ERR_INVALID_ARG, "max_launches %lld out of range [0, 2^20]", (long long)max_launches);
  {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev), "get device");
    if (dev != h->device) return fail(WAN_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  }
  release_events(h);
  h->att_ev.reserve(2 * max_launches);
  for (int64_t i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t e;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      release_events(h);
      return fail(WAN_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    h->att_ev.push_back(e);
  }
  return WAN_OK;
}

extern "C" wan_status wan_dit_attention_time(wan_dit* h, double* total_ms, int64_t* launches) {
  g_err.clear();
  if (!h || !total_ms || !launches) return fail(WAN_ERR_INVALID_ARG, "handle or output pointer is NULL");
  {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev), "get device");
    if (dev != h->device) return fail(WAN_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  }
  double t = 0.0;
  for (int64_t i = 0; i < h->att_used; ++i) {
    HIP_TRY(hipEventSynchronize(h->att_ev[2 * i + 1]), "attention timing: wait");
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, h->att_ev[2 * i], h->att_ev[2 * i + 1]), "attention timing: elapsed");
    t += ms;
  }
  *total_ms = t;
  *launches = h->att_used;
  h->att_used = 0;
  return WAN_OK;
}

extern "C" wan_status wan_dit_create(const wan_dit_config* cfg, const wan_weight* weights, size_t n_weights,
                                     void* hip_stream, wan_dit** out) {
  g_err.clear();
  if (!out) return fail(WAN_ERR_INVALID_ARG, "out handle pointer is NULL");
  *out = nullptr;
  wan_status st = check_config(cfg);
  if (st != WAN_OK) return st;
  if (!weights && n_weights) return fail(WAN_ERR_INVALID_ARG, "weights is NULL");

  // ---- match names and shapes
  const std::vector<Expect> exp = expected_weights(*cfg);
  std::unordered_map<std::string, size_t> by_name;
  for (size_t i = 0; i < n_weights; ++i) {
    const wan_weight& w = weights[i];
    if (!w.name) return fail(WAN_ERR_INVALID_ARG, "weight %zu has no name", i);
    if (!by_name.emplace(w.name, i).second) return fail(WAN_ERR_MISSING_WEIGHT, "weight %s given twice", w.name);
  }
  for (const Expect& e : exp) {
    auto it = by_name.find(e.name);
    if (it == by_name.end()) return fail(WAN_ERR_MISSING_WEIGHT, "missing weight %s", e.name.c_str());
    const wan_weight& w = weights[it->second];
    if (w.dtype != WAN_F32 && w.dtype != WAN_BF16) return fail(WAN_ERR_DTYPE, "weight %s: bad dtype", e.name.c_str());
    bool ok = w.ndim == (int)e.shape.size();
    for (int d = 0; ok && d < w.ndim; ++d) ok = w.shape[d] == e.shape[d];
    if (!ok)
      return fail(WAN_ERR_SHAPE, "weight %s has shape %s, expected %s", e.name.c_str(), shape_str(w.shape, w.ndim).c_str(),
                  shape_str(e.shape.data(), (int)e.shape.size()).c_str());
    if (!w.data) return fail(WAN_ERR_INVALID_ARG, "weight %s: data is NULL", e.name.c_str());
  }
  if (by_name.size() != exp.size()) {
    std::unordered_map<std::string, int> want;
    for (const Expect& e : exp) want[e.name] = 1;
    for (auto& kv : by_name)
      if (!want.count(kv.first)) return fail(WAN_ERR_MISSING_WEIGHT, "unexpected weight %s", kv.first.c_str());
  }

  // ---- allocate
  wan_dit* h = new wan_dit();
  h->cfg = *cfg;
  (void)hipGetDevice(&h->device);
  h->kp_pe = round_up(4LL * cfg->in_channels, 64);
  h->n_out = 4LL * cfg->out_channels;
  h->kp_img = cfg->max_image_len > 0 ? round_up(cfg->image_dim, 64) : 0;
  Arena plan_w, plan_ws;
  plan_weights(h, plan_w);
  plan_workspace(h, plan_ws);
  h->wbytes = plan_w.used;
  h->wsbytes = plan_ws.used;
  if (hipMalloc(&h->wmem, h->wbytes) != hipSuccess) {
    (void)hipGetLastError();
    free_handle(h);
    return fail(WAN_ERR_OOM, "could not allocate %zu bytes of packed weights", plan_w.used);
  }
  if (hipMalloc(&h->wsmem, h->wsbytes) != hipSuccess) {
    (void)hipGetLastError();
    free_handle(h);
    return fail(WAN_ERR_OOM, "could not allocate %zu bytes of workspace", plan_ws.used);
  }
  Arena aw{(char*)h->wmem, h->wbytes, 0}, aws{(char*)h->wsmem, h->wsbytes, 0};
  plan_weights(h, aw);
  plan_workspace(h, aws);

  // ---- pack
  hipStream_t s = (hipStream_t)hip_stream;
  auto W = [&](const std::string& n) -> const wan_weight& { return weights[by_name.at(n)]; };
  auto pack_lin = [&](const std::string& n, bf16_t* dst, int64_t rows, int64_t cols, int64_t ldd) {
    const wan_weight& w = W(n);
    return launch_pack_bf16(w.data, w.dtype, rows, cols, cols, dst, ldd, s);
  };
  auto pack_f = [&](const std::string& n, float* dst) {
    const wan_weight& w = W(n);
    return launch_pack_f32(w.data, w.dtype, numel(w.shape, w.ndim), dst, s);
  };
  const int64_t D = cfg->dim, Fd = cfg->ffn_dim;
  hipError_t e = hipSuccess;
  auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
  chk(pack_lin("patch_embedding.weight", h->w_pe, D, 4LL * cfg->in_channels, h->kp_pe));
  chk(pack_f("patch_embedding.bias", h->b_pe));
  chk(pack_f("time_embedder.linear_1.weight", h->t_w1)); chk(pack_f("time_embedder.linear_1.bias", h->t_b1));
  chk(pack_f("time_embedder.linear_2.weight", h->t_w2)); chk(pack_f("time_embedder.linear_2.bias", h->t_b2));
  chk(pack_f("time_proj.weight", h->t_wp)); chk(pack_f("time_proj.bias", h->t_bp));
  chk(pack_lin("text_embedder.linear_1.weight", h->c_w1, D, cfg->text_dim, cfg->text_dim));
  chk(pack_f("text_embedder.linear_1.bias", h->c_b1));
  chk(pack_lin("text_embedder.linear_2.weight", h->c_w2, D, D, D));
  chk(pack_f("text_embedder.linear_2.bias", h->c_b2));
  if (cfg->max_image_len > 0) {
    chk(pack_lin("image_embedder.linear_1.weight", h->i_w1, D, cfg->image_dim, h->kp_img));
    chk(pack_f("image_embedder.linear_1.bias", h->i_b1));
    chk(pack_lin("image_embedder.linear_2.weight", h->i_w2, D, D, D));
    chk(pack_f("image_embedder.linear_2.bias", h->i_b2));
  }
  for (int k = 0; k < cfg->num_layers; ++k) {
    const std::string p = "blocks." + std::to_string(k) + ".";
    BlockW& b = h->blocks[k];
    chk(pack_lin(p + "attn1.to_q.weight", b.wqkv, D, D, D));
    chk(pack_lin(p + "attn1.to_k.weight", b.wqkv + D * D, D, D, D));
    chk(pack_lin(p + "attn1.to_v.weight", b.wqkv + 2 * D * D, D, D, D));
    chk(pack_f(p + "attn1.to_q.bias", b.bqkv));
    chk(pack_f(p + "attn1.to_k.bias", b.bqkv + D));
    chk(pack_f(p + "attn1.to_v.bias", b.bqkv + 2 * D));
    chk(pack_lin(p + "attn1.to_out.weight", b.wo, D, D, D)); chk(pack_f(p + "attn1.to_out.bias", b.bo));
    chk(pack_lin(p + "attn2.to_q.weight", b.wq2, D, D, D)); chk(pack_f(p + "attn2.to_q.bias", b.bq2));
    chk(pack_lin(p + "attn2.to_k.weight", b.wkv2, D, D, D));
    chk(pack_lin(p + "attn2.to_v.weight", b.wkv2 + D * D, D, D, D));
    chk(pack_f(p + "attn2.to_k.bias", b.bkv2));
    chk(pack_f(p + "attn2.to_v.bias", b.bkv2 + D));
    chk(pack_lin(p + "attn2.to_out.weight", b.wo2, D, D, D)); chk(pack_f(p + "attn2.to_out.bias", b.bo2));
    chk(pack_lin(p + "ffn.proj_in.weight", b.w1, Fd, D, D)); chk(pack_f(p + "ffn.proj_in.bias", b.b1));
    chk(pack_lin(p + "ffn.proj_out.weight", b.w2, D, Fd, Fd)); chk(pack_f(p + "ffn.proj_out.bias", b.b2));
    chk(pack_f(p + "attn1.norm_q.weight", b.gq)); chk(pack_f(p + "attn1.norm_k.weight", b.gk));
    chk(pack_f(p + "attn2.norm_q.weight", b.gq2)); chk(pack_f(p + "attn2.norm_k.weight", b.gk2));
    chk(pack_f(p + "norm2.weight", b.n2w)); chk(pack_f(p + "norm2.bias", b.n2b));
    chk(pack_f(p + "scale_shift_table", b.table));
    if (cfg->max_image_len > 0) {
      chk(pack_lin(p + "attn2.add_k_proj.weight", b.wkvi, D, D, D));
      chk(pack_lin(p + "attn2.add_v_proj.weight", b.wkvi + D * D, D, D, D));
      chk(pack_f(p + "attn2.add_k_proj.bias", b.bkvi));
      chk(pack_f(p + "attn2.add_v_proj.bias", b.bkvi + D));
      chk(pack_f(p + "attn2.norm_added_k.weight", b.gki));
    }
  }
  chk(pack_f("scale_shift_table", h->head_table));
  chk(pack_lin("proj_out.weight", h->w_out, h->n_out, D, D));
  chk(pack_f("proj_out.bias", h->b_out));
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free_handle(h);
    return fail(WAN_ERR_HIP, "weight packing failed: %s", hipGetErrorString(e));
  }
  *out = h;
  return WAN_OK;
}

namespace {

// One forward's inputs after validation.  dup: the latent, timestep and image tensors hold batch element 0
// only, used for every batch element (the CFG pair of a denoising step).
struct FwdIn {
  int64_t B, Cin, F, Hz, Wz, Fp, Hp, Wp, L, Lt, Li;
  const void* latent; int lat_dtype;
  const float* t; bool per_tok;
  const void* text; int text_dtype;
  const void* image; int image_dtype;   // image == nullptr: no image tokens
  bool dup;
};

// How the proj_out values leave: unpatchified into out, or (denoising step) CFG-combined and Euler-stepped.
struct FwdOut {
  void* out; int dtype;
  bool step; float scale, sigma, sigma_next;
};

wan_status check_device(const wan_dit* h) {
  int dev = -1;
  (void)hipGetDevice(&dev);
  if (dev != h->device) return fail(WAN_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  return WAN_OK;
}

// Validate latent / timestep / text (and image) against the configuration; B_in is the batch the tensors
// hold (1 for a denoising step), in.B the batch the forward runs.
wan_status check_inputs(const wan_dit* h, const wan_tensor* latent, const wan_tensor* timestep, const wan_tensor* text,
                        const wan_tensor* image, int64_t B_in, int64_t B_text, FwdIn& in) {
  wan_status st;
  if ((st = check_tensor(latent, "latent")) != WAN_OK) return st;
  if ((st = check_tensor(timestep, "timestep")) != WAN_OK) return st;
  if ((st = check_tensor(text, "text_emb")) != WAN_OK) return st;
  if (image && (st = check_tensor(image, "image_emb")) != WAN_OK) return st;
  const wan_dit_config& c = h->cfg;
  if (latent->ndim != 5) return fail(WAN_ERR_SHAPE, "latent must be [B, C, F, H, W]");
  in.Cin = latent->shape[1]; in.F = latent->shape[2]; in.Hz = latent->shape[3]; in.Wz = latent->shape[4];
  if (B_in < 0 ? false : latent->shape[0] != B_in)
    return fail(WAN_ERR_SHAPE, "latent batch must be %lld, got %lld", (long long)B_in, (long long)latent->shape[0]);
  const int64_t B = latent->shape[0];
  if (in.Cin != c.in_channels)
    return fail(WAN_ERR_SHAPE, "latent has %lld channels, config expects %d", (long long)in.Cin, c.in_channels);
  if (in.Hz % 2 || in.Wz % 2)
    return fail(WAN_ERR_SHAPE, "latent height and width must be even (got %lld x %lld)", (long long)in.Hz, (long long)in.Wz);
  in.Fp = in.F; in.Hp = in.Hz / 2; in.Wp = in.Wz / 2; in.L = in.Fp * in.Hp * in.Wp;
  if (in.Fp > 1024 || in.Hp > 1024 || in.Wp > 1024)
    return fail(WAN_ERR_SHAPE, "token grid %lldx%lldx%lld exceeds the 1024 rotary positions per axis", (long long)in.Fp,
                (long long)in.Hp, (long long)in.Wp);
  if (in.B > c.max_batch) return fail(WAN_ERR_SHAPE, "batch %lld > max_batch %lld", (long long)in.B, (long long)c.max_batch);
  if (in.L > c.max_tokens) return fail(WAN_ERR_SHAPE, "%lld tokens > max_tokens %lld", (long long)in.L, (long long)c.max_tokens);
  // timestep
  if (timestep->dtype != WAN_F32) return fail(WAN_ERR_DTYPE, "timestep must be WAN_F32");
  if (timestep->ndim == 1 && timestep->shape[0] == B) in.per_tok = false;
  else if (timestep->ndim == 2 && timestep->shape[0] == B && timestep->shape[1] == in.L) in.per_tok = true;
  else return fail(WAN_ERR_SHAPE, "timestep must be [B] or [B, L] (B=%lld, L=%lld), got %s", (long long)B, (long long)in.L,
                   shape_str(timestep->shape, timestep->ndim).c_str());
  if (in.per_tok && !c.per_token_timestep)
    return fail(WAN_ERR_UNSUPPORTED, "per-token timesteps need per_token_timestep = 1 in the config");
  // text
  if (text->ndim != 3 || text->shape[0] != B_text || text->shape[2] != c.text_dim)
    return fail(WAN_ERR_SHAPE, "text_emb must be [%lld, Lt, %d], got %s", (long long)B_text, c.text_dim,
                shape_str(text->shape, text->ndim).c_str());
  in.Lt = text->shape[1];
  if (in.B > 0 && (in.Lt < 1 || in.Lt > c.max_text_len))
    return fail(WAN_ERR_SHAPE, "text length %lld outside [1, %lld]", (long long)in.Lt, (long long)c.max_text_len);
  if (text->dtype == WAN_BF16 && ((uintptr_t)text->data & 15)) return fail(WAN_ERR_INVALID_ARG, "bf16 text_emb must be 16-byte aligned");
  // image tokens
  in.Li = 0;
  in.image = nullptr;
  if (image) {
    if (c.max_image_len == 0) return fail(WAN_ERR_UNSUPPORTED, "image tokens need max_image_len > 0 in the config");
    if (image->ndim != 3 || image->shape[0] != B || image->shape[2] != c.image_dim)
      return fail(WAN_ERR_SHAPE, "image_emb must be [%lld, Li, %d], got %s", (long long)B, c.image_dim,
                  shape_str(image->shape, image->ndim).c_str());
    in.Li = image->shape[1];
    if (in.B > 0 && (in.Li < 1 || in.Li > c.max_image_len))
      return fail(WAN_ERR_SHAPE, "image length %lld outside [1, %lld]", (long long)in.Li, (long long)c.max_image_len);
    if (image->dtype == WAN_BF16 && ((uintptr_t)image->data & 15))
      return fail(WAN_ERR_INVALID_ARG, "bf16 image_emb must be 16-byte aligned");
    in.image = image->data;
    in.image_dtype = image->dtype;
  }
  in.latent = latent->data; in.lat_dtype = latent->dtype;
  in.t = (const float*)timestep->data;
  in.text = text->data; in.text_dtype = text->dtype;
  return check_device(h);
}

// Enqueue one forward (forward sequence in the file header).
wan_status enqueue_forward(wan_dit* h, const FwdIn& in, const FwdOut& fo, hipStream_t s) {
  const wan_dit_config& c = h->cfg;
  const int64_t B = in.B, L = in.L, Lt = in.Lt, Li = in.Li, F = in.F, Hz = in.Hz, Wz = in.Wz;
  const int64_t D = c.dim, Fd = c.ffn_dim, M = B * L, nh = c.num_heads;
  const int64_t R = in.per_tok ? M : B;
  const int64_t rows_per_mod = in.per_tok ? 1 : L;
  const int dt = c.rope_dim_t, dh = c.rope_dim_h, dw = c.rope_dim_w;
  const int64_t ldv = round_up(L, 64), ldv2 = round_up(Lt, 64), ldvi = round_up(Li, 64);
  const float eps = c.eps, qs = attention_q_scale();

  // 1. patch embedding -> fp32 residual stream x [M, D]
  if (in.dup) {
    for (int64_t b = 0; b < B; ++b)
      HIP_TRY(launch_patchify(in.latent, in.lat_dtype, 1, in.Cin, F, Hz, Wz, h->kp_pe, h->P + b * L * h->kp_pe, s), "patchify");
  } else {
    HIP_TRY(launch_patchify(in.latent, in.lat_dtype, B, in.Cin, F, Hz, Wz, h->kp_pe, h->P, s), "patchify");
  }
  HIP_TRY(launch_gemm_bf16(h->P, h->kp_pe, h->w_pe, h->kp_pe, h->b_pe, M, D, h->kp_pe, EPI_F32, h->x, D, nullptr, nullptr,
                           0, 1, s), "patch embed");
  // 2. timestep embedding (fp32)
  const float* t = in.t;
  if (in.dup) {
    const int64_t per = in.per_tok ? L : 1;
    for (int64_t b = 0; b < B; ++b)
      HIP_TRY(hipMemcpyAsync(h->t_dup + b * per, in.t, per * sizeof(float), hipMemcpyDeviceToDevice, s), "timestep copy");
    t = h->t_dup;
  }
  HIP_TRY(launch_sinusoid(t, R, c.freq_dim, h->t_s, s), "sinusoid");
  HIP_TRY(launch_gemm_f32(h->t_s, c.freq_dim, h->t_w1, c.freq_dim, h->t_b1, R, D, c.freq_dim, h->t_h, D, 0, 1, s), "time linear_1");
  HIP_TRY(launch_gemm_f32(h->t_h, D, h->t_w2, D, h->t_b2, R, D, D, h->temb, D, 0, 0, s), "time linear_2");
  HIP_TRY(launch_gemm_f32(h->temb, D, h->t_wp, D, h->t_bp, R, 6 * D, D, h->tproj, 6 * D, 1, 0, s), "time_proj");
  // 3. text projection
  const bf16_t* txt = (const bf16_t*)in.text;
  if (in.text_dtype == WAN_F32) {
    HIP_TRY(launch_pack_bf16(in.text, WAN_F32, B * Lt, c.text_dim, c.text_dim, h->text_bf, c.text_dim, s), "text cast");
    txt = h->text_bf;
  }
  HIP_TRY(launch_gemm_bf16(txt, c.text_dim, h->c_w1, c.text_dim, h->c_b1, B * Lt, D, c.text_dim, EPI_GELU_BF16, h->ctx_h, D,
                           nullptr, nullptr, 0, 1, s), "text linear_1");
  HIP_TRY(launch_gemm_bf16(h->ctx_h, D, h->c_w2, D, h->c_b2, B * Lt, D, D, EPI_BF16, h->ctx, D, nullptr, nullptr, 0, 1, s),
          "text linear_2");
  // 3b. image tokens: the same two-layer projection on the CLIP features (batch element 0 copied for dup)
  if (Li > 0) {
    const int64_t rows_in = in.dup ? Li : B * Li;
    HIP_TRY(launch_pack_bf16(in.image, in.image_dtype, rows_in, c.image_dim, c.image_dim, h->img_bf, h->kp_img, s), "image cast");
    if (in.dup)
      for (int64_t b = 1; b < B; ++b)
        HIP_TRY(hipMemcpyAsync(h->img_bf + b * Li * h->kp_img, h->img_bf, Li * h->kp_img * sizeof(bf16_t),
                               hipMemcpyDeviceToDevice, s), "image copy");
    HIP_TRY(launch_gemm_bf16(h->img_bf, h->kp_img, h->i_w1, h->kp_img, h->i_b1, B * Li, D, h->kp_img, EPI_GELU_BF16, h->img_h,
                             D, nullptr, nullptr, 0, 1, s), "image linear_1");
    HIP_TRY(launch_gemm_bf16(h->img_h, D, h->i_w2, D, h->i_b2, B * Li, D, D, EPI_BF16, h->img_ctx, D, nullptr, nullptr, 0, 1, s),
            "image linear_2");
  }
  // 4. rotary tables for this grid
  HIP_TRY(launch_rope_table(h->rope, (int)in.Fp, (int)in.Hp, (int)in.Wp, dt, dh, dw, c.rope_theta, s), "rope table");

  // 5. blocks.  res_* describe the pending residual: the previous block's FFN output and its gate.
  //    Queries leave the QK norm multiplied by the attention's log2(e)/sqrt(128).
  int res_mode = 0;
  const float* res_tab = nullptr;
  const float* res_src = nullptr;
  for (int k = 0; k < c.num_layers; ++k) {
    const BlockW& b = h->blocks[k];
    // self-attention
    HIP_TRY(launch_layernorm(h->x, M, D, eps, 0, b.table + 0 * D, b.table + 1 * D, h->tproj, 6 * D, 0 * D, 1 * D,
                             rows_per_mod, nullptr, nullptr, res_mode, h->br, res_tab, res_src, 6 * D, h->y, s), "norm1");
    HIP_TRY(launch_gemm_bf16(h->y, D, b.wqkv, D, b.bqkv, M, 3 * D, D, EPI_BF16, h->qkv, 3 * D, nullptr, nullptr, 0, 1, s,
                             h->gemm_ws, h->gemm_ws_bytes), "qkv");
    HIP_TRY(launch_rms_rope(h->qkv, 3 * D, M, D, eps, 0, b.gq, D, b.gk, h->rope, L, (int)in.Fp, (int)in.Hp, (int)in.Wp, dt, dh,
                            dw, s, qs), "qk norm rope");
    HIP_TRY(launch_transpose_v(h->qkv, 3 * D, 2 * D, B, L, (int)nh, h->vt, ldv, s), "v transpose");
    const bool timed = 2 * h->att_used < (int64_t)h->att_ev.size();
    if (timed) HIP_TRY(hipEventRecord(h->att_ev[2 * h->att_used], s), "self attention timing");
    HIP_TRY(launch_attention(h->qkv, 3 * D, h->qkv + D, 3 * D, h->vt, ldv, h->attn, D, B, L, L, (int)nh, true, s,
                             h->attn_ws, h->attn_ws_bytes, true), "self attention");
    if (timed) HIP_TRY(hipEventRecord(h->att_ev[2 * h->att_used++ + 1], s), "self attention timing");
    HIP_TRY(launch_gemm_bf16(h->attn, D, b.wo, D, b.bo, M, D, D, EPI_BF16, h->br, D, nullptr, nullptr, 0, 1, s,
                             h->gemm_ws, h->gemm_ws_bytes), "attn1 out");
    // cross-attention: x += gate1 * attn, then norm2 (affine)
    HIP_TRY(launch_layernorm(h->x, M, D, eps, 1, nullptr, nullptr, nullptr, 0, 0, 0, rows_per_mod, b.n2w, b.n2b, 2, h->br,
                             b.table + 2 * D, h->tproj + 2 * D, 6 * D, h->y, s), "norm2");
    bf16_t* q2 = h->qkv;
    HIP_TRY(launch_gemm_bf16(h->y, D, b.wq2, D, b.bq2, M, D, D, EPI_BF16, q2, D, nullptr, nullptr, 0, 1, s,
                             h->gemm_ws, h->gemm_ws_bytes), "q2");
    HIP_TRY(launch_rms_rope(q2, D, M, D, eps, 0, b.gq2, 0, nullptr, nullptr, L, 1, 1, 1, dt, dh, dw, s, qs), "q2 norm");
    HIP_TRY(launch_gemm_bf16(h->ctx, D, b.wkv2, D, b.bkv2, B * Lt, 2 * D, D, EPI_BF16, h->kv2, 2 * D, nullptr, nullptr, 0, 1, s),
            "kv2");
    HIP_TRY(launch_rms_rope(h->kv2, 2 * D, B * Lt, D, eps, 0, b.gk2, 0, nullptr, nullptr, Lt, 1, 1, 1, dt, dh, dw, s), "k2 norm");
    HIP_TRY(launch_transpose_v(h->kv2, 2 * D, D, B, Lt, (int)nh, h->vt2, ldv2, s), "v2 transpose");
    HIP_TRY(launch_attention(q2, D, h->kv2, 2 * D, h->vt2, ldv2, h->attn, D, B, L, Lt, (int)nh, false, s, h->attn_ws,
                             h->attn_ws_bytes, true), "cross attention");
    if (Li > 0) {
      // the image tokens' own keys and values; their attention output is added to the text one
      HIP_TRY(launch_gemm_bf16(h->img_ctx, D, b.wkvi, D, b.bkvi, B * Li, 2 * D, D, EPI_BF16, h->kvi, 2 * D, nullptr, nullptr, 0,
                               1, s), "image kv");
      HIP_TRY(launch_rms_rope(h->kvi, 2 * D, B * Li, D, eps, 0, b.gki, 0, nullptr, nullptr, Li, 1, 1, 1, dt, dh, dw, s),
              "image k norm");
      HIP_TRY(launch_transpose_v(h->kvi, 2 * D, D, B, Li, (int)nh, h->vti, ldvi, s), "image v transpose");
      HIP_TRY(launch_attention(q2, D, h->kvi, 2 * D, h->vti, ldvi, h->attn, D, B, L, Li, (int)nh, false, s, h->attn_ws,
                               h->attn_ws_bytes, true, true), "image cross attention");
    }
    HIP_TRY(launch_gemm_bf16(h->attn, D, b.wo2, D, b.bo2, M, D, D, EPI_BF16, h->br, D, nullptr, nullptr, 0, 1, s,
                             h->gemm_ws, h->gemm_ws_bytes), "attn2 out");
    // feed-forward: x += cross-attn (ungated), then norm3 + modulation
    HIP_TRY(launch_layernorm(h->x, M, D, eps, 0, b.table + 3 * D, b.table + 4 * D, h->tproj, 6 * D, 3 * D, 4 * D,
                             rows_per_mod, nullptr, nullptr, 1, h->br, nullptr, nullptr, 0, h->y, s), "norm3");
    HIP_TRY(launch_gemm_bf16(h->y, D, b.w1, D, b.b1, M, Fd, D, EPI_GELU_BF16, h->hbuf, Fd, nullptr, nullptr, 0, 1, s,
                             h->gemm_ws, h->gemm_ws_bytes), "ffn1");
    HIP_TRY(launch_gemm_bf16(h->hbuf, Fd, b.w2, Fd, b.b2, M, D, Fd, EPI_BF16, h->br, D, nullptr, nullptr, 0, 1, s,
                             h->gemm_ws, h->gemm_ws_bytes), "ffn2");
    res_mode = 2;
    res_tab = b.table + 5 * D;
    res_src = h->tproj + 5 * D;
  }

  // 6. output head: x += gate2 * ffn of the last block, then norm_out + (table + temb) modulation
  HIP_TRY(launch_layernorm(h->x, M, D, eps, 0, h->head_table, h->head_table + D, h->temb, D, 0, 0, rows_per_mod, nullptr,
                           nullptr, res_mode, h->br, res_tab, res_src, 6 * D, h->y, s), "norm_out");
  HIP_TRY(launch_gemm_bf16(h->y, D, h->w_out, D, h->b_out, M, h->n_out, D, EPI_F32, h->z, h->n_out, nullptr, nullptr, 0, 1, s),
          "proj_out");
  if (fo.step)
    HIP_TRY(launch_cfg_euler(h->z, h->n_out, c.out_channels, F, Hz, Wz, in.latent, fo.dtype, fo.scale, fo.sigma,
                             fo.sigma_next, fo.out, s), "cfg + euler step");
  else
    HIP_TRY(launch_unpatchify(h->z, h->n_out, B, c.out_channels, F, Hz, Wz, fo.out, fo.dtype, s), "unpatchify");
  return WAN_OK;
}

wan_status forward_common(wan_dit* h, const wan_tensor* latent, const wan_tensor* timestep, const wan_tensor* text,
                          const wan_tensor* image, wan_tensor* out, void* hip_stream) {
  if (!h) return fail(WAN_ERR_INVALID_ARG, "handle is NULL");
  wan_status st;
  if ((st = check_tensor(latent, "latent")) != WAN_OK) return st;
  if ((st = check_tensor(out, "out")) != WAN_OK) return st;
  FwdIn in;
  in.B = latent->ndim == 5 ? latent->shape[0] : 0;
  in.dup = false;
  if ((st = check_inputs(h, latent, timestep, text, image, -1, in.B, in)) != WAN_OK) return st;
  const wan_dit_config& c = h->cfg;
  if (out->ndim != 5 || out->shape[0] != in.B || out->shape[1] != c.out_channels || out->shape[2] != in.F ||
      out->shape[3] != in.Hz || out->shape[4] != in.Wz)
    return fail(WAN_ERR_SHAPE, "out must be [B, %d, F, H, W] matching the latent, got %s", c.out_channels,
                shape_str(out->shape, out->ndim).c_str());
  if (out->dtype != latent->dtype) return fail(WAN_ERR_DTYPE, "out dtype must match the latent dtype");
  if (in.B == 0 || in.L == 0) return WAN_OK;
  FwdOut fo{out->data, out->dtype, false, 0.f, 0.f, 0.f};
  return enqueue_forward(h, in, fo, (hipStream_t)hip_stream);
}

}  // namespace

extern "C" wan_status wan_dit_forward(wan_dit* h, const wan_tensor* latent, const wan_tensor* timestep,
                                      const wan_tensor* text, wan_tensor* out, void* hip_stream) {
  g_err.clear();
  return forward_common(h, latent, timestep, text, nullptr, out, hip_stream);
}

extern "C" wan_status wan_dit_forward_image(wan_dit* h, const wan_tensor* latent, const wan_tensor* timestep,
                                            const wan_tensor* text, const wan_tensor* image, wan_tensor* out,
                                            void* hip_stream) {
  g_err.clear();
  if (!image) return fail(WAN_ERR_INVALID_ARG, "image_emb is NULL (use wan_dit_forward without image tokens)");
  return forward_common(h, latent, timestep, text, image, out, hip_stream);
}

extern "C" wan_status wan_dit_denoise_step(wan_dit* h, const wan_tensor* latent, const wan_tensor* timestep,
                                           const wan_tensor* text_pair, const wan_tensor* image, float guidance_scale,
                                           float sigma, float sigma_next, wan_tensor* x_next, void* hip_stream) {
  g_err.clear();
  if (!h) return fail(WAN_ERR_INVALID_ARG, "handle is NULL");
  wan_status st;
  if ((st = check_tensor(x_next, "x_next")) != WAN_OK) return st;
  if (!std::isfinite(guidance_scale) || !std::isfinite(sigma) || !std::isfinite(sigma_next))
    return fail(WAN_ERR_INVALID_ARG, "guidance_scale, sigma and sigma_next must be finite");
  if (h->cfg.max_batch < 2) return fail(WAN_ERR_UNSUPPORTED, "a denoising step runs a batch of 2: max_batch must be >= 2");
  FwdIn in;
  in.B = 2;
  in.dup = true;
  if ((st = check_inputs(h, latent, timestep, text_pair, image, 1, 2, in)) != WAN_OK) return st;
  const wan_dit_config& c = h->cfg;
  if (x_next->ndim != 5 || x_next->shape[0] != 1 || x_next->shape[1] != c.out_channels || x_next->shape[2] != in.F ||
      x_next->shape[3] != in.Hz || x_next->shape[4] != in.Wz)
    return fail(WAN_ERR_SHAPE, "x_next must be [1, %d, F, H, W] matching the latent, got %s", c.out_channels,
                shape_str(x_next->shape, x_next->ndim).c_str());
  if (x_next->dtype != latent->dtype) return fail(WAN_ERR_DTYPE, "x_next dtype must match the latent dtype");
  if (x_next->data == latent->data) return fail(WAN_ERR_INVALID_ARG, "x_next must not alias the latent");
  if (in.L == 0) return WAN_OK;
  FwdOut fo{x_next->data, x_next->dtype, true, guidance_scale, sigma, sigma_next};
  return enqueue_forward(h, in, fo, (hipStream_t)hip_stream);
}

// =====================================================================================================
// Per-stage entry points
// =====================================================================================================

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

extern "C" wan_status wan_op_patchify(const void* latent, int32_t dtype, int64_t B, int64_t C, int64_t F, int64_t Hz,
                                      int64_t Wz, int64_t kp, void* p, void* stream) {
  g_err.clear();
  REQUIRE(dtype == WAN_F32 || dtype == WAN_BF16, WAN_ERR_DTYPE, "patchify: bad dtype");
  REQUIRE(B >= 0 && C > 0 && F >= 0 && Hz >= 0 && Wz >= 0, WAN_ERR_SHAPE, "patchify: bad sizes");
  REQUIRE(Hz % 2 == 0 && Wz % 2 == 0, WAN_ERR_SHAPE, "patchify: H and W must be even");
  REQUIRE(kp >= 4 * C && kp % 8 == 0, WAN_ERR_SHAPE, "patchify: kp must be >= 4C and a multiple of 8");
  REQUIRE((latent && p) || B * F * Hz * Wz == 0, WAN_ERR_INVALID_ARG, "patchify: NULL pointer");
  HIP_TRY(launch_patchify(latent, dtype, B, C, F, Hz, Wz, kp, (bf16_t*)p, (hipStream_t)stream), "patchify");
  return WAN_OK;
}

extern "C" wan_status wan_op_unpatchify(const float* z, int64_t ldz, int64_t B, int64_t C, int64_t F, int64_t Hz, int64_t Wz,
                                        void* out, int32_t out_dtype, void* stream) {
  g_err.clear();
  REQUIRE(out_dtype == WAN_F32 || out_dtype == WAN_BF16, WAN_ERR_DTYPE, "unpatchify: bad dtype");
  REQUIRE(B >= 0 && C > 0 && F >= 0 && Hz >= 0 && Wz >= 0 && Hz % 2 == 0 && Wz % 2 == 0, WAN_ERR_SHAPE, "unpatchify: bad sizes");
  REQUIRE(ldz >= 4 * C, WAN_ERR_SHAPE, "unpatchify: ldz < 4C");
  REQUIRE((z && out) || B * F * Hz * Wz == 0, WAN_ERR_INVALID_ARG, "unpatchify: NULL pointer");
  HIP_TRY(launch_unpatchify(z, ldz, B, C, F, Hz, Wz, out, out_dtype, (hipStream_t)stream), "unpatchify");
  return WAN_OK;
}

extern "C" wan_status wan_op_cfg_euler(const float* z, int64_t ldz, int64_t C, int64_t F, int64_t Hz, int64_t Wz,
                                       const void* x, int64_t Cx, int32_t dtype, float guidance_scale, float sigma,
                                       float sigma_next, void* x_next, void* stream) {
  g_err.clear();
  REQUIRE(dtype == WAN_F32 || dtype == WAN_BF16, WAN_ERR_DTYPE, "cfg_euler: bad dtype");
  REQUIRE(C > 0 && Cx >= C && F >= 0 && Hz >= 0 && Wz >= 0 && Hz % 2 == 0 && Wz % 2 == 0, WAN_ERR_SHAPE, "cfg_euler: bad sizes");
  REQUIRE(ldz >= 4 * C, WAN_ERR_SHAPE, "cfg_euler: ldz < 4C");
  REQUIRE((z && x && x_next) || F * Hz * Wz == 0, WAN_ERR_INVALID_ARG, "cfg_euler: NULL pointer");
  REQUIRE(x != x_next || F * Hz * Wz == 0, WAN_ERR_INVALID_ARG, "cfg_euler: x_next must not alias x");
  REQUIRE(std::isfinite(guidance_scale) && std::isfinite(sigma) && std::isfinite(sigma_next), WAN_ERR_INVALID_ARG,
          "cfg_euler: guidance_scale, sigma and sigma_next must be finite");
  HIP_TRY(launch_cfg_euler(z, ldz, C, F, Hz, Wz, x, dtype, guidance_scale, sigma, sigma_next, x_next, (hipStream_t)stream),
          "cfg_euler");
  return WAN_OK;
}

// Argument checks shared by wan_op_gemm and wan_op_gemm_ws.
static wan_status check_gemm(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias, int64_t M,
                             int64_t N, int64_t K, int32_t epilogue, void* out, int64_t ldo, const float* gate_tab,
                             const float* gate_src, int64_t gate_ld, int64_t rows_per_gate) {
  REQUIRE(epilogue >= 0 && epilogue <= 4, WAN_ERR_INVALID_ARG, "gemm: bad epilogue %d", epilogue);
  REQUIRE(M >= 0 && N > 0 && K > 0, WAN_ERR_SHAPE, "gemm: bad sizes");
  REQUIRE(K % 64 == 0, WAN_ERR_SHAPE, "gemm: K must be a multiple of 64");
  REQUIRE(N % 4 == 0, WAN_ERR_SHAPE, "gemm: N must be a multiple of 4");
  REQUIRE(ldx >= K && ldw >= K && ldx % 8 == 0 && ldw % 8 == 0, WAN_ERR_SHAPE, "gemm: ldx/ldw must be >= K and multiples of 8");
  REQUIRE(ldo >= N && ldo % 4 == 0, WAN_ERR_SHAPE, "gemm: ldo must be >= N and a multiple of 4");
  REQUIRE(x && w && bias && out, WAN_ERR_INVALID_ARG, "gemm: NULL pointer");
  REQUIRE(epilogue != EPI_GATE_F32 || (gate_tab && gate_src && rows_per_gate > 0 && gate_ld >= N), WAN_ERR_INVALID_ARG,
          "gemm: gate epilogue needs gate_tab, gate_src, gate_ld >= N and rows_per_gate > 0");
  return WAN_OK;
}

extern "C" wan_status wan_op_gemm(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias, int64_t M,
                                  int64_t N, int64_t K, int32_t epilogue, void* out, int64_t ldo, const float* gate_tab,
                                  const float* gate_src, int64_t gate_ld, int64_t rows_per_gate, void* stream) {
  g_err.clear();
  const wan_status st = check_gemm(x, ldx, w, ldw, bias, M, N, K, epilogue, out, ldo, gate_tab, gate_src, gate_ld,
                                   rows_per_gate);
  if (st != WAN_OK) return st;
  HIP_TRY(launch_gemm_bf16((const bf16_t*)x, ldx, (const bf16_t*)w, ldw, bias, M, N, K, epilogue, out, ldo, gate_tab, gate_src,
                           gate_ld, rows_per_gate, (hipStream_t)stream), "gemm");
  return WAN_OK;
}

extern "C" int64_t wan_op_gemm_workspace_bytes(void) { return gemm_workspace_bytes(); }

extern "C" wan_status wan_op_gemm_ws(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias, int64_t M,
                                     int64_t N, int64_t K, int32_t epilogue, void* out, int64_t ldo, const float* gate_tab,
                                     const float* gate_src, int64_t gate_ld, int64_t rows_per_gate, void* workspace,
                                     int64_t workspace_bytes, void* stream) {
  g_err.clear();
  const wan_status st = check_gemm(x, ldx, w, ldw, bias, M, N, K, epilogue, out, ldo, gate_tab, gate_src, gate_ld,
                                   rows_per_gate);
  if (st != WAN_OK) return st;
  REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 15) == 0 && workspace_bytes >= gemm_workspace_bytes(),
          WAN_ERR_INVALID_ARG, "gemm_ws: workspace must be 16-byte aligned and >= %lld bytes",
          (long long)gemm_workspace_bytes());
  HIP_TRY(launch_gemm_bf16((const bf16_t*)x, ldx, (const bf16_t*)w, ldw, bias, M, N, K, epilogue, out, ldo, gate_tab, gate_src,
                           gate_ld, rows_per_gate, (hipStream_t)stream, (float*)workspace, workspace_bytes), "gemm_ws");
  return WAN_OK;
}

extern "C" wan_status wan_op_layernorm(float* x, int64_t rows, int64_t D, float eps, int32_t mode, const float* tab_shift,
                                       const float* tab_scale, const float* src, int64_t src_ld, int64_t src_shift_off,
                                       int64_t src_scale_off, int64_t rows_per_src, const float* gamma, const float* beta,
                                       int32_t res_mode, const void* res, const float* res_tab, const float* res_src,
                                       int64_t res_ld, void* y, void* stream) {
  g_err.clear();
  REQUIRE(rows >= 0 && D % 256 == 0 && D > 0 && D <= 6144, WAN_ERR_SHAPE, "layernorm: D must be a multiple of 256 <= 6144");
  REQUIRE(mode == 0 || mode == 1, WAN_ERR_INVALID_ARG, "layernorm: mode must be 0 or 1");
  REQUIRE(res_mode >= 0 && res_mode <= 2, WAN_ERR_INVALID_ARG, "layernorm: res_mode must be 0, 1 or 2");
  REQUIRE(x && y, WAN_ERR_INVALID_ARG, "layernorm: NULL pointer");
  REQUIRE(rows_per_src > 0, WAN_ERR_INVALID_ARG, "layernorm: rows_per_src must be positive");
  if (mode == 0)
    REQUIRE(tab_shift && tab_scale && src && src_ld % 4 == 0 && src_shift_off % 4 == 0 && src_scale_off % 4 == 0,
            WAN_ERR_INVALID_ARG, "layernorm: modulation sources missing or misaligned");
  else
    REQUIRE(gamma && beta, WAN_ERR_INVALID_ARG, "layernorm: affine mode needs gamma and beta");
  if (res_mode) REQUIRE(res, WAN_ERR_INVALID_ARG, "layernorm: residual mode needs the branch output");
  if (res_mode == 2)
    REQUIRE(res_tab && res_src && res_ld % 4 == 0, WAN_ERR_INVALID_ARG, "layernorm: gated residual needs res_tab, res_src");
  HIP_TRY(launch_layernorm(x, rows, D, eps, mode, tab_shift, tab_scale, src, src_ld, src_shift_off, src_scale_off, rows_per_src,
                           gamma, beta, res_mode, (const bf16_t*)res, res_tab, res_src, res_ld, (bf16_t*)y,
                           (hipStream_t)stream), "layernorm");
  return WAN_OK;
}

extern "C" int64_t wan_op_rope_table_floats(int32_t Fp, int32_t Hp, int32_t Wp, int32_t dt, int32_t dh, int32_t dw) {
  return rope_table_floats(Fp, Hp, Wp, dt, dh, dw);
}

extern "C" wan_status wan_op_rope_table(float* table, int32_t Fp, int32_t Hp, int32_t Wp, int32_t dt, int32_t dh, int32_t dw,
                                        double theta, void* stream) {
  g_err.clear();
  REQUIRE(table, WAN_ERR_INVALID_ARG, "rope_table: NULL table");
  REQUIRE(Fp > 0 && Hp > 0 && Wp > 0 && Fp <= 1024 && Hp <= 1024 && Wp <= 1024, WAN_ERR_SHAPE, "rope_table: grid out of range");
  REQUIRE(dt > 0 && dh > 0 && dw > 0 && !((dt | dh | dw) & 1) && dt + dh + dw == 128, WAN_ERR_SHAPE,
          "rope_table: dims must be even and sum to 128");
  HIP_TRY(launch_rope_table(table, Fp, Hp, Wp, dt, dh, dw, theta, (hipStream_t)stream), "rope_table");
  return WAN_OK;
}

extern "C" wan_status wan_op_qk_norm_rope(void* buf, int64_t ld, int64_t rows, int64_t D, float eps, int64_t off_a,
                                          const float* gamma_a, int64_t off_b, const float* gamma_b, const float* table,
                                          int64_t L, int32_t Fp, int32_t Hp, int32_t Wp, int32_t dt, int32_t dh, int32_t dw,
                                          float scale_a, void* stream) {
  g_err.clear();
  REQUIRE(rows >= 0 && D > 0 && D % 512 == 0 && D <= 12288, WAN_ERR_SHAPE, "qk_norm_rope: D must be a multiple of 512 <= 12288");
  REQUIRE(buf && gamma_a, WAN_ERR_INVALID_ARG, "qk_norm_rope: NULL pointer");
  REQUIRE(ld % 8 == 0 && off_a % 8 == 0 && off_b % 8 == 0 && off_a + D <= ld && (!gamma_b || off_b + D <= ld), WAN_ERR_SHAPE,
          "qk_norm_rope: segments must be 8-aligned and inside the row");
  if (table) {
    REQUIRE(L > 0 && (int64_t)Fp * Hp * Wp == L, WAN_ERR_SHAPE, "qk_norm_rope: L must equal Fp*Hp*Wp");
    REQUIRE(dt > 0 && dh > 0 && dw > 0 && !((dt | dh | dw) & 1) && dt + dh + dw == 128, WAN_ERR_SHAPE,
            "qk_norm_rope: rope dims must be even and sum to 128");
  }
  REQUIRE(std::isfinite(scale_a), WAN_ERR_INVALID_ARG, "qk_norm_rope: scale_a must be finite");
  HIP_TRY(launch_rms_rope((bf16_t*)buf, ld, rows, D, eps, off_a, gamma_a, off_b, gamma_b, table, L, Fp, Hp, Wp, dt, dh, dw,
                          (hipStream_t)stream, scale_a), "qk_norm_rope");
  return WAN_OK;
}

extern "C" wan_status wan_op_transpose_v(const void* src, int64_t ld, int64_t col_off, int64_t B, int64_t L, int32_t nh,
                                         void* vt, int64_t ldv, void* stream) {
  g_err.clear();
  REQUIRE(B >= 0 && L >= 0 && nh > 0, WAN_ERR_SHAPE, "transpose_v: bad sizes");
  REQUIRE(ldv % 64 == 0 && ldv >= L, WAN_ERR_SHAPE, "transpose_v: ldv must be a multiple of 64 and >= L");
  REQUIRE(ld % 8 == 0 && col_off % 8 == 0 && col_off + 128LL * nh <= ld, WAN_ERR_SHAPE, "transpose_v: bad row layout");
  REQUIRE((src && vt) || B == 0, WAN_ERR_INVALID_ARG, "transpose_v: NULL pointer");
  HIP_TRY(launch_transpose_v((const bf16_t*)src, ld, col_off, B, L, nh, (bf16_t*)vt, ldv, (hipStream_t)stream), "transpose_v");
  return WAN_OK;
}

extern "C" wan_status wan_op_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt, int64_t ldv,
                                       void* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int32_t nh, void* stream) {
  g_err.clear();
  REQUIRE(B >= 0 && Lq >= 0 && nh > 0, WAN_ERR_SHAPE, "attention: bad sizes");
  REQUIRE(Lkv >= 1 || B * Lq == 0, WAN_ERR_SHAPE, "attention: at least one key is needed");
  REQUIRE(ldv % 64 == 0 && ldv >= Lkv, WAN_ERR_SHAPE, "attention: ldv must be a multiple of 64 and >= Lkv");
  REQUIRE(ldq % 8 == 0 && ldk % 8 == 0 && ldo % 4 == 0 && ldq >= 128LL * nh && ldk >= 128LL * nh && ldo >= 128LL * nh,
          WAN_ERR_SHAPE, "attention: bad row strides");
  REQUIRE((q && k && vt && o) || B * Lq == 0, WAN_ERR_INVALID_ARG, "attention: NULL pointer");
  HIP_TRY(launch_attention((const bf16_t*)q, ldq, (const bf16_t*)k, ldk, (const bf16_t*)vt, ldv, (bf16_t*)o, ldo, B, Lq, Lkv, nh,
                           Lq == Lkv, (hipStream_t)stream), "attention");
  return WAN_OK;
}

extern "C" int64_t wan_op_attention_workspace_bytes(int64_t B, int64_t Lq, int32_t nh) {
  if (B < 0 || Lq < 0 || nh <= 0) return -1;
  return attention_workspace_bytes(B, Lq, nh);
}

extern "C" wan_status wan_op_attention_ws(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                                          int64_t ldv, void* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int32_t nh,
                                          void* workspace, int64_t workspace_bytes, void* stream) {
  g_err.clear();
  REQUIRE(B >= 0 && Lq >= 0 && nh > 0, WAN_ERR_SHAPE, "attention: bad sizes");
  REQUIRE(Lkv >= 1 || B * Lq == 0, WAN_ERR_SHAPE, "attention: at least one key is needed");
  REQUIRE(ldv % 64 == 0 && ldv >= Lkv, WAN_ERR_SHAPE, "attention: ldv must be a multiple of 64 and >= Lkv");
  REQUIRE(ldq % 8 == 0 && ldk % 8 == 0 && ldo % 4 == 0 && ldq >= 128LL * nh && ldk >= 128LL * nh && ldo >= 128LL * nh,
          WAN_ERR_SHAPE, "attention: bad row strides");
  REQUIRE((q && k && vt && o) || B * Lq == 0, WAN_ERR_INVALID_ARG, "attention: NULL pointer");
  REQUIRE(workspace != nullptr && ((uintptr_t)workspace & 15) == 0 &&
              workspace_bytes >= attention_workspace_bytes(B, Lq, nh),
          WAN_ERR_INVALID_ARG, "attention: workspace must be 16-byte aligned and >= %lld bytes",
          (long long)attention_workspace_bytes(B, Lq, nh));
  HIP_TRY(launch_attention((const bf16_t*)q, ldq, (const bf16_t*)k, ldk, (const bf16_t*)vt, ldv, (bf16_t*)o, ldo, B, Lq, Lkv, nh,
                           Lq == Lkv, (hipStream_t)stream, (float*)workspace, workspace_bytes), "attention");
  return WAN_OK;
}

extern "C" wan_status wan_op_attention_noalloc(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                                                int64_t ldv, void* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv,
                                                int32_t nh, void* stream) {
  g_err.clear();
  REQUIRE(B >= 0 && Lq >= 0 && nh > 0, WAN_ERR_SHAPE, "attention: bad sizes");
  REQUIRE(Lkv >= 1 || B * Lq == 0, WAN_ERR_SHAPE, "attention: at least one key is needed");
  REQUIRE(ldv % 64 == 0 && ldv >= Lkv, WAN_ERR_SHAPE, "attention: ldv must be a multiple of 64 and >= Lkv");
  REQUIRE(ldq % 8 == 0 && ldk % 8 == 0 && ldo % 4 == 0 && ldq >= 128LL * nh && ldk >= 128LL * nh && ldo >= 128LL * nh,
          WAN_ERR_SHAPE, "attention: bad row strides");
  REQUIRE((q && k && vt && o) || B * Lq == 0, WAN_ERR_INVALID_ARG, "attention: NULL pointer");
  const int64_t units = B * nh * ceil_div(Lq, 256);
  REQUIRE(units <= attention_scratch_max_units(), WAN_ERR_UNSUPPORTED,
          "attention_noalloc: %lld (batch, head, 256-query) units exceed the static workspace's %lld",
          (long long)units, (long long)attention_scratch_max_units());
  HIP_TRY(launch_attention_noalloc((const bf16_t*)q, ldq, (const bf16_t*)k, ldk, (const bf16_t*)vt, ldv, (bf16_t*)o, ldo, B,
                                   Lq, Lkv, nh, (hipStream_t)stream), "attention_noalloc");
  return WAN_OK;
}

extern "C" wan_status wan_op_time_embed(const float* t, int64_t rows, int32_t freq_dim, int64_t D, const float* w1,
                                        const float* b1, const float* w2, const float* b2, const float* wp, const float* bp,
                                        float* temb, float* tproj, float* work, void* stream) {
  g_err.clear();
  REQUIRE(rows >= 0 && freq_dim > 0 && freq_dim % 2 == 0 && D > 0, WAN_ERR_SHAPE, "time_embed: bad sizes");
  REQUIRE((t && w1 && b1 && w2 && b2 && wp && bp && temb && tproj && work) || rows == 0, WAN_ERR_INVALID_ARG,
          "time_embed: NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  float* sbuf = work;
  float* hb = work + rows * freq_dim;
  HIP_TRY(launch_sinusoid(t, rows, freq_dim, sbuf, s), "sinusoid");
  HIP_TRY(launch_gemm_f32(sbuf, freq_dim, w1, freq_dim, b1, rows, D, freq_dim, hb, D, 0, 1, s), "time linear_1");
  HIP_TRY(launch_gemm_f32(hb, D, w2, D, b2, rows, D, D, temb, D, 0, 0, s), "time linear_2");
  HIP_TRY(launch_gemm_f32(temb, D, wp, D, bp, rows, 6 * D, D, tproj, 6 * D, 1, 0, s), "time_proj");
  return WAN_OK;
}

extern "C" wan_status wan_probe_mfma(float* sink, int32_t blocks, int64_t rounds, int32_t random_operands,
                                     void* stream) {
  g_err.clear();
  REQUIRE(blocks > 0 && rounds > 0, WAN_ERR_SHAPE, "probe_mfma: blocks and rounds must be positive");
  REQUIRE(sink, WAN_ERR_INVALID_ARG, "probe_mfma: NULL sink");
  HIP_TRY(launch_mfma_probe(sink, blocks, rounds, random_operands, (hipStream_t)stream), "mfma probe");
  return WAN_OK;
}
