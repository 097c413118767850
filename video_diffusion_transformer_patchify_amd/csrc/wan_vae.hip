// Host orchestrator and C ABI of the Wan-VAE causal decoder: weight validation and packing, the frame
// caches, and the per-chunk launch sequence.
//
// Decode (diffusers WanPipeline notes page, section "vae.decode"): post_quant_conv over the latent,
// then WanDecoder3d on the first latent frame alone and on the later frames chunk by chunk; every causal
// convolution sees its input sequence through a feature cache of the last 2 input frames, so the
// result is the causal convolution over the whole sequence.  Per chunk:
//   prep (un-normalise + post_quant_conv) -> conv_in
//   stage A (H x W, 4b ch):   mid block (2 residual blocks), up block 0 (3), upsample3d
//   stage B (2H x 2W):        up block 1 (3, the first with a 1x1x1 shortcut 2b -> 4b), upsample3d
//   stage C (4H x 4W, 2b ch): up block 2 (3), upsample2d
//   stage D (8H x 8W, b ch):  up block 3 (3), RMS_norm + SiLU, conv_out (clamped, into the video)
// Residual block: norm1 + SiLU -> conv1 -> norm2 + SiLU -> conv2 with the residual added in its epilogue.
//
// Frame caches.  Each causal convolution's input lives in a ring of 2 + (frames per chunk) padded frames:
// the 2 newest frames of earlier chunks, then the current chunk's frames, which the producing kernel
// writes in place.  After the chunk the ring turns so that its 2 newest frames become the next chunk's
// history: no frame is copied.  Time tap dt of output frame j reads ring position hist + j - 2 + dt, or
// the zero frame before the first frame.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <unordered_map>
#include <vector>

#include "common.h"
#include "launch.h"
#include "launch_vae.h"
#include "wan_vae.h"

namespace {

thread_local std::string g_verr;

wan_status vfail(wan_status st, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_verr = buf;
  return st;
}

#define VREQ(cond, st, ...)                  \
  do {                                       \
    if (!(cond)) return vfail(st, __VA_ARGS__); \
  } while (0)

#define VHIP(expr, what)                                                                      \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return vfail(WAN_ERR_HIP, "%s: %s", what, hipGetErrorString(e_));   \
  } while (0)

int64_t cpad(int64_t c) { return (c + 15) / 16 * 16; }
int ncf_for(int64_t cout) { return cout % 96 == 0 ? 3 : 1; }

struct Arena {
  char* base = nullptr;
  size_t used = 0;
  template <typename T>
  T* take(int64_t count) {
    size_t bytes = ((size_t)count * sizeof(T) + 255) & ~(size_t)255;
    T* p = (T*)(base ? base + used : nullptr);
    used += bytes;
    return p;
  }
};

struct ConvW {
  bf16_t* w = nullptr;
  float* b = nullptr;
  int64_t cin = 0, cout = 0;
  int kt = 1, ks = 1, ncf = 1;
  int64_t ntiles() const { return (cout + 32 * ncf - 1) / (32 * ncf); }
};

struct ResW {
  std::string name;
  int stage;               // 0..3 = A..D
  int64_t ci, co;
  float *g1 = nullptr, *g2 = nullptr;
  ConvW c1, c2, sc;
  bool has_sc = false;
};

struct UpW {
  std::string name;
  bool time;
  int64_t ci, co;
  ConvW tc, rs;
};

// Ring of padded frames holding a causal convolution's input: hist frames of history, then n current.
struct Seq {
  bf16_t* base = nullptr;
  int64_t cap_elems = 0;   // elements reserved per frame (the largest frame size)
  int R = 0, head = 0, hist = 0;
  int64_t c = 0;           // channels (padded to 16)
  bf16_t* slot(int pos, int64_t fe) const { return base + (int64_t)((head + pos) % R) * fe; }
  void end(int n) {
    const int nh = hist + n < 2 ? hist + n : 2;
    head = (head + hist + n - nh) % R;
    hist = nh;
  }
  void reset() { head = hist = 0; }
};

}  // namespace

struct wan_vae {
  wan_vae_config cfg;
  int device = 0;
  void* wmem = nullptr;
  void* amem = nullptr;
  size_t wbytes = 0, abytes = 0;
  float *mean, *stdv, *wq, *bq;
  ConvW conv_in, conv_out;
  float* g_out;
  std::vector<ResW> res;   // 14, forward order
  UpW up[3];
  // activations
  Seq pq, xa, xb, nout;
  std::vector<Seq> n1, n2;   // per residual block
  bf16_t *ha, *hb, *hc, *hd, *ta, *tb, *ub, *xc, *xd, *zero;
  int64_t cur_h = -1, cur_w = -1;
  // opt-in timing of the 3x3x3 causal convolutions with 96-channel tiles (wan_vae_time_convs)
  std::vector<hipEvent_t> ev;
  int64_t ev_used = 0;
  double ev_flops = 0.0;
};

namespace {

void release_events(wan_vae* h) {
  for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
  h->ev.clear();
  h->ev_used = 0;
  h->ev_flops = 0.0;
}

void free_vae(wan_vae* h) {
  if (!h) return;
  release_events(h);
  if (h->wmem) (void)hipFree(h->wmem);
  if (h->amem) (void)hipFree(h->amem);
  delete h;
}

struct Expect {
  std::string name;
  std::vector<int64_t> shape;
};

// The decoder's residual blocks and upsamplers in forward order (widths from the base width b).
void build_layout(wan_vae* h) {
  const int64_t b = h->cfg.base_dim, A = 4 * b, Bc = 4 * b, C = 2 * b, D = b;
  auto add = [&](const std::string& n, int stage, int64_t ci, int64_t co) {
    ResW r;
    r.name = n;
    r.stage = stage;
    r.ci = ci;
    r.co = co;
    r.has_sc = ci != co;
    h->res.push_back(r);
  };
  for (int j = 0; j < 2; ++j) add("decoder.mid_block.resnets." + std::to_string(j), 0, A, A);
  for (int j = 0; j < 3; ++j) add("decoder.up_blocks.0.resnets." + std::to_string(j), 0, A, A);
  add("decoder.up_blocks.1.resnets.0", 1, A / 2, Bc);
  for (int j = 1; j < 3; ++j) add("decoder.up_blocks.1.resnets." + std::to_string(j), 1, Bc, Bc);
  for (int j = 0; j < 3; ++j) add("decoder.up_blocks.2.resnets." + std::to_string(j), 2, C, C);
  for (int j = 0; j < 3; ++j) add("decoder.up_blocks.3.resnets." + std::to_string(j), 3, D, D);
  h->up[0] = UpW{"decoder.up_blocks.0.upsamplers.0", true, A, A / 2, {}, {}};
  h->up[1] = UpW{"decoder.up_blocks.1.upsamplers.0", true, Bc, Bc / 2, {}, {}};
  h->up[2] = UpW{"decoder.up_blocks.2.upsamplers.0", false, C, C / 2, {}, {}};
}

std::vector<Expect> expected(const wan_vae* h) {
  const int64_t z = h->cfg.z_dim, b = h->cfg.base_dim;
  std::vector<Expect> e = {{"latents_mean", {z}}, {"latents_std", {z}}, {"post_quant_conv.weight", {z, z, 1, 1, 1}},
                           {"post_quant_conv.bias", {z}}, {"decoder.conv_in.weight", {4 * b, z, 3, 3, 3}},
                           {"decoder.conv_in.bias", {4 * b}}};
  for (const ResW& r : h->res) {
    e.push_back({r.name + ".norm1.gamma", {r.ci}});
    e.push_back({r.name + ".conv1.weight", {r.co, r.ci, 3, 3, 3}});
    e.push_back({r.name + ".conv1.bias", {r.co}});
    e.push_back({r.name + ".norm2.gamma", {r.co}});
    e.push_back({r.name + ".conv2.weight", {r.co, r.co, 3, 3, 3}});
    e.push_back({r.name + ".conv2.bias", {r.co}});
    if (r.has_sc) {
      e.push_back({r.name + ".conv_shortcut.weight", {r.co, r.ci, 1, 1, 1}});
      e.push_back({r.name + ".conv_shortcut.bias", {r.co}});
    }
  }
  for (const UpW& u : h->up) {
    if (u.time) {
      e.push_back({u.name + ".time_conv.weight", {2 * u.ci, u.ci, 3, 1, 1}});
      e.push_back({u.name + ".time_conv.bias", {2 * u.ci}});
    }
    e.push_back({u.name + ".resample.1.weight", {u.co, u.ci, 3, 3}});
    e.push_back({u.name + ".resample.1.bias", {u.co}});
  }
  e.push_back({"decoder.norm_out.gamma", {b}});
  e.push_back({"decoder.conv_out.weight", {3, b, 3, 3, 3}});
  e.push_back({"decoder.conv_out.bias", {3}});
  return e;
}

std::string shape_str(const int64_t* s, int n) {
  std::string o = "[";
  for (int i = 0; i < n; ++i) o += (i ? "," : "") + std::to_string(s[i]);
  return o + "]";
}

void plan_conv(Arena& a, ConvW& c, int64_t cin, int64_t cout, int kt, int ks) {
  c.cin = cin;
  c.cout = cout;
  c.kt = kt;
  c.ks = ks;
  c.ncf = ncf_for(cout);
  c.w = a.take<bf16_t>(vae_packed_conv_elems(cout, cin, kt, ks, c.ncf));
  c.b = a.take<float>(c.ntiles() * 32 * c.ncf);
}

void plan_weights(wan_vae* h, Arena& a) {
  const int64_t z = h->cfg.z_dim, b = h->cfg.base_dim;
  h->mean = a.take<float>(z);
  h->stdv = a.take<float>(z);
  h->wq = a.take<float>(z * z);
  h->bq = a.take<float>(z);
  plan_conv(a, h->conv_in, z, 4 * b, 3, 3);
  for (ResW& r : h->res) {
    r.g1 = a.take<float>(cpad(r.ci));
    r.g2 = a.take<float>(cpad(r.co));
    plan_conv(a, r.c1, r.ci, r.co, 3, 3);
    plan_conv(a, r.c2, r.co, r.co, 3, 3);
    if (r.has_sc) plan_conv(a, r.sc, r.ci, r.co, 1, 1);
  }
  for (UpW& u : h->up) {
    if (u.time) plan_conv(a, u.tc, u.ci, 2 * u.ci, 3, 1);
    plan_conv(a, u.rs, u.ci, u.co, 1, 3);
  }
  h->g_out = a.take<float>(cpad(b));
  plan_conv(a, h->conv_out, b, 3, 3, 3);
}

void plan_seq(Arena& a, Seq& s, int64_t c, int64_t H, int64_t W, int R) {
  s.c = cpad(c);
  s.cap_elems = vae_frame_elems(s.c, H, W);
  s.R = R;
  s.base = a.take<bf16_t>(s.cap_elems * R);
}

void plan_acts(wan_vae* h, Arena& a) {
  const int64_t b = h->cfg.base_dim, H = h->cfg.max_height, W = h->cfg.max_width;
  const int c = h->cfg.chunk_frames;
  const int nA = c, nB = 2 * c, nD = 4 * c;
  const int64_t hs[4] = {H, 2 * H, 4 * H, 8 * H}, ws[4] = {W, 2 * W, 4 * W, 8 * W};
  const int nfr[4] = {nA, nB, nD, nD};
  plan_seq(a, h->pq, h->cfg.z_dim, H, W, 2 + nA);
  plan_seq(a, h->xa, 4 * b, H, W, 2 + nA);
  plan_seq(a, h->xb, 4 * b, hs[1], ws[1], 2 + nB);
  plan_seq(a, h->nout, b, hs[3], ws[3], 2 + nD);
  h->n1.assign(h->res.size(), Seq());
  h->n2.assign(h->res.size(), Seq());
  for (size_t i = 0; i < h->res.size(); ++i) {
    const ResW& r = h->res[i];
    plan_seq(a, h->n1[i], r.ci, hs[r.stage], ws[r.stage], 2 + nfr[r.stage]);
    plan_seq(a, h->n2[i], r.co, hs[r.stage], ws[r.stage], 2 + nfr[r.stage]);
  }
  h->ha = a.take<bf16_t>(vae_frame_elems(4 * b, H, W) * nA);
  h->ta = a.take<bf16_t>(vae_frame_elems(4 * b, H, W) * 2 * nA);
  h->ub = a.take<bf16_t>(vae_frame_elems(cpad(2 * b), hs[1], ws[1]) * nB);
  h->hb = a.take<bf16_t>(vae_frame_elems(4 * b, hs[1], ws[1]) * nB);
  h->tb = a.take<bf16_t>(vae_frame_elems(4 * b, hs[1], ws[1]) * 2 * nB);
  h->xc = a.take<bf16_t>(vae_frame_elems(cpad(2 * b), hs[2], ws[2]) * nD);
  h->hc = a.take<bf16_t>(vae_frame_elems(cpad(2 * b), hs[2], ws[2]) * nD);
  h->xd = a.take<bf16_t>(vae_frame_elems(cpad(b), hs[3], ws[3]) * nD);
  h->hd = a.take<bf16_t>(vae_frame_elems(cpad(b), hs[3], ws[3]) * nD);
  // the zero frame stands in for causal padding: as large as any convolution input frame
  int64_t zmax = vae_frame_elems(cpad(h->cfg.z_dim), H, W);
  for (int st = 0; st < 4; ++st) {
    const int64_t cmax = st < 2 ? 4 * b : (st == 2 ? 2 * b : b);
    const int64_t e = vae_frame_elems(cpad(cmax), hs[st], ws[st]);
    if (e > zmax) zmax = e;
  }
  h->zero = a.take<bf16_t>(zmax);
}

// ---- launch helpers ---------------------------------------------------------------------------------

struct Ctx {
  wan_vae* h;
  hipStream_t s;
  int64_t H[4], W[4];        // current stage sizes
  hipError_t err = hipSuccess;
  void chk(hipError_t e) { if (err == hipSuccess) err = e; }
  int64_t fe(int64_t c, int st) const { return vae_frame_elems(cpad(c), H[st], W[st]); }
};

// KT = 3 inputs of output frame j from a ring; positions before the first frame read the zero frame.
void ring_inputs(const Ctx& x, const Seq& q, int st, int n, VaeConvArgs& a) {
  const int64_t fe = vae_frame_elems(q.c, x.H[st], x.W[st]);
  for (int j = 0; j < n; ++j)
    for (int dt = 0; dt < 3; ++dt) {
      const int pos = q.hist + j - 2 + dt;
      a.in[j][dt] = pos < 0 ? x.h->zero : q.slot(pos, fe);
    }
}

void conv_launch(Ctx& x, const ConvW& c, VaeConvArgs& a, int st_out, int nf, int up, int split, bool video) {
  a.w = c.w;
  a.bias = c.b;
  a.nf = nf;
  a.H = (int32_t)x.H[st_out];
  a.W = (int32_t)x.W[st_out];
  a.Hin = up ? a.H / 2 : a.H;
  a.Win = up ? a.W / 2 : a.W;
  a.cin_blocks = (int32_t)(cpad(c.cin) / 16);
  a.split = split;
  a.cpart = (int32_t)(split == 2 ? c.cout / 2 : cpad(c.cout));
  a.ntiles = (int32_t)c.ntiles();
  a.tiles_x = (a.W + 31) / 32;
  a.tiles_y = (a.H + 15) / 16;
  wan_vae* h = x.h;
  const bool timed = h && !video && c.kt == 3 && c.ks == 3 && c.ncf == 3 && h->ev_used + 2 <= (int64_t)h->ev.size();
  if (timed) x.chk(hipEventRecord(h->ev[h->ev_used], x.s));
  x.chk(launch_vae_conv(a, c.kt, c.ks, up, c.ncf, video, x.s));
  if (timed) {
    x.chk(hipEventRecord(h->ev[h->ev_used + 1], x.s));
    h->ev_used += 2;
    h->ev_flops += 2.0 * (double)c.cout * (double)c.cin * 27.0 * nf * (double)a.H * (double)a.W;
  }
}

void norm_launch(Ctx& x, const bf16_t* const* in, bf16_t* const* out, int nf, int64_t c, int st, const float* g) {
  x.chk(launch_vae_rms_silu(in, out, nf, c, cpad(c) / 16, x.H[st], x.W[st], g, x.h->cfg.eps, x.s));
}

// A convolution whose one output-channel tile holds all of its channels (stage D: 96 channels in one
// workgroup) applies the RMS norm + SiLU that follows it in its own epilogue.
bool fusable(const ConvW& c) { return c.cout == 32 * c.ncf && c.ntiles() == 1; }

void fuse_norm(const Ctx& x, VaeConvArgs& a, bf16_t* const* nout, int n, const float* g, bool only) {
  for (int j = 0; j < n; ++j) a.nout[j] = nout[j];
  a.ngamma = g;
  a.neps = x.h->cfg.eps;
  a.nonly = only ? 1 : 0;
}

// Slots of the current frames in ring q at stage st.
void ring_slots(const Ctx& x, const Seq& q, int st, int n, bf16_t** dst) {
  const int64_t fe = vae_frame_elems(q.c, x.H[st], x.W[st]);
  for (int j = 0; j < n; ++j) dst[j] = q.slot(q.hist + j, fe);
}

// One residual block on n frames: in[j] -> out[j] (in == out unless the block has a shortcut).
// in_normed: the producer of `in` already wrote norm1's output into this block's first ring.  next_g,
// next_nout: the norm that follows the block (the next block's norm1 or the head's), applied in conv2's
// epilogue where it can be; the return value says whether it was.
bool res_block(Ctx& x, size_t i, bf16_t* const* in, bf16_t* const* out, bf16_t* hbuf, int n, bool in_normed = false,
               const float* next_g = nullptr, bf16_t* const* next_nout = nullptr) {
  wan_vae* h = x.h;
  const ResW& r = h->res[i];
  Seq& q1 = h->n1[i];
  Seq& q2 = h->n2[i];
  const int st = r.stage;
  const int64_t fe1 = vae_frame_elems(q1.c, x.H[st], x.W[st]);
  const int64_t fe2 = vae_frame_elems(q2.c, x.H[st], x.W[st]);
  const int64_t feh = x.fe(r.co, st);
  bf16_t* p1[VAE_MAXF];
  bf16_t* p2[VAE_MAXF];
  bf16_t* ph[VAE_MAXF];
  for (int j = 0; j < n; ++j) {
    p1[j] = q1.slot(q1.hist + j, fe1);
    p2[j] = q2.slot(q2.hist + j, fe2);
    ph[j] = hbuf + j * feh;
  }
  if (!in_normed) norm_launch(x, in, p1, n, r.ci, st, r.g1);
  VaeConvArgs a1{};
  ring_inputs(x, q1, st, n, a1);
  for (int j = 0; j < n; ++j) a1.out[j] = ph[j];
  const bool fuse1 = fusable(r.c1);
  if (fuse1) fuse_norm(x, a1, p2, n, r.g2, true);   // conv1's output is only norm2's input
  conv_launch(x, r.c1, a1, st, n, 0, 1, false);
  if (!fuse1) norm_launch(x, ph, p2, n, r.co, st, r.g2);
  if (r.has_sc) {
    VaeConvArgs as{};
    for (int j = 0; j < n; ++j) {
      as.in[j][0] = in[j];
      as.out[j] = out[j];
    }
    conv_launch(x, r.sc, as, st, n, 0, 1, false);
  }
  VaeConvArgs a2{};
  ring_inputs(x, q2, st, n, a2);
  for (int j = 0; j < n; ++j) {
    a2.out[j] = out[j];
    a2.res[j] = out[j];
  }
  const bool fuse2 = next_nout != nullptr && fusable(r.c2);
  if (fuse2) fuse_norm(x, a2, next_nout, n, next_g, false);
  conv_launch(x, r.c2, a2, st, n, 0, 1, false);
  return fuse2;
}

// upsample3d / upsample2d of n input frames at stage st: time conv (not on the first chunk), then the
// nearest x2 + 3x3 conv into dst frames at stage st + 1.  next_g, next_nout: the norm that follows,
// applied in that conv's epilogue where it can be (*normed says whether it was).
int upsample(Ctx& x, const UpW& u, Seq* ring, bf16_t* const* in, int n, int st, bool first, bf16_t* tbuf,
             bf16_t* const* dst, const float* next_g = nullptr, bf16_t* const* next_nout = nullptr,
             bool* normed = nullptr) {
  const bf16_t* src[2 * VAE_MAXF];
  int m = n;
  if (u.time && !first) {
    VaeConvArgs at{};
    ring_inputs(x, *ring, st, n, at);
    const int64_t fe = x.fe(u.ci, st);
    for (int j = 0; j < 2 * n; ++j) at.out[j] = tbuf + j * fe;
    conv_launch(x, u.tc, at, st, n, 0, 2, false);
    m = 2 * n;
    for (int j = 0; j < m; ++j) src[j] = tbuf + j * fe;
  } else {
    for (int j = 0; j < n; ++j) src[j] = in[j];
  }
  VaeConvArgs ar{};
  for (int j = 0; j < m; ++j) {
    ar.in[j][0] = src[j];
    ar.out[j] = dst[j];
  }
  const bool fuse = next_nout != nullptr && fusable(u.rs);
  if (fuse) fuse_norm(x, ar, next_nout, m, next_g, false);
  conv_launch(x, u.rs, ar, st + 1, m, 1, 1, false);
  if (normed) *normed = fuse;
  return m;
}

// One decoder call on latent frames [f0, f0 + n) of one sample (n = 1 for the first chunk).
void decode_chunk(Ctx& x, const void* z, int zdt, int64_t F, int64_t f0, int n, bool first, void* video,
                  int vdt, int64_t T, int64_t t0) {
  wan_vae* h = x.h;
  const int64_t b = h->cfg.base_dim;
  const int nB = first ? 1 : 2 * n, nD = first ? 1 : 4 * n;
  bf16_t* pa[VAE_MAXF];
  bf16_t* pb[VAE_MAXF];
  bf16_t* pc[VAE_MAXF];
  bf16_t* pd[VAE_MAXF];
  bf16_t* pu[VAE_MAXF];
  // prep -> pq ring
  {
    const int64_t fe = vae_frame_elems(h->pq.c, x.H[0], x.W[0]);
    for (int j = 0; j < n; ++j) pa[j] = h->pq.slot(h->pq.hist + j, fe);
    x.chk(launch_vae_prep(z, zdt, F, x.H[0], x.W[0], f0, n, h->mean, h->stdv, h->wq, h->bq, pa, x.s));
  }
  // conv_in -> xa ring (current frames)
  {
    const int64_t fe = vae_frame_elems(h->xa.c, x.H[0], x.W[0]);
    for (int j = 0; j < n; ++j) pa[j] = h->xa.slot(h->xa.hist + j, fe);
    VaeConvArgs a{};
    ring_inputs(x, h->pq, 0, n, a);
    for (int j = 0; j < n; ++j) a.out[j] = pa[j];
    conv_launch(x, h->conv_in, a, 0, n, 0, 1, false);
  }
  size_t ri = 0;
  for (; ri < 5; ++ri) res_block(x, ri, pa, pa, h->ha, n);                     // mid block + up block 0
  for (int j = 0; j < nB; ++j) pu[j] = h->ub + j * x.fe(2 * b, 1);
  upsample(x, h->up[0], &h->xa, pa, n, 0, first, h->ta, pu);
  {
    const int64_t fe = vae_frame_elems(h->xb.c, x.H[1], x.W[1]);
    for (int j = 0; j < nB; ++j) pb[j] = h->xb.slot(h->xb.hist + j, fe);
  }
  res_block(x, ri++, pu, pb, h->hb, nB);                                     // up block 1, with shortcut
  for (; ri < 8; ++ri) res_block(x, ri, pb, pb, h->hb, nB);
  for (int j = 0; j < nD; ++j) pc[j] = h->xc + j * x.fe(2 * b, 2);
  upsample(x, h->up[1], &h->xb, pb, nB, 1, first, h->tb, pc);
  for (; ri < 11; ++ri) res_block(x, ri, pc, pc, h->hc, nD);                 // up block 2
  for (int j = 0; j < nD; ++j) pd[j] = h->xd + j * x.fe(b, 3);
  // stage D: each norm runs in the epilogue of the convolution before it (96 channels per workgroup)
  bf16_t* pn[VAE_MAXF];
  ring_slots(x, h->n1[ri], 3, nD, pn);
  bool normed = false;
  upsample(x, h->up[2], nullptr, pc, nD, 2, first, nullptr, pd, h->res[ri].g1, pn, &normed);
  for (; ri < 14; ++ri) {                                                     // up block 3
    const bool last = ri + 1 == 14;
    ring_slots(x, last ? h->nout : h->n1[ri + 1], 3, nD, pn);
    normed = res_block(x, ri, pd, pd, h->hd, nD, normed, last ? h->g_out : h->res[ri + 1].g1, pn);
  }
  // head: RMS_norm + SiLU -> conv_out into the video frames t0 .. t0 + nD - 1
  {
    bf16_t* po[VAE_MAXF];
    ring_slots(x, h->nout, 3, nD, po);
    if (!normed) norm_launch(x, pd, po, nD, b, 3, h->g_out);
    VaeConvArgs a{};
    ring_inputs(x, h->nout, 3, nD, a);
    a.video = video;
    a.video_T = (int32_t)T;
    a.video_bf16 = vdt == WAN_BF16;
    for (int j = 0; j < nD; ++j) a.video_t[j] = (int32_t)(t0 + j);
    conv_launch(x, h->conv_out, a, 3, nD, 0, 1, true);
  }
  // turn the rings: the 2 newest frames become the history; the first latent frame does not enter the
  // time convs' history (their rings are the stage-A / stage-B residual streams)
  h->pq.end(n);
  h->xa.end(n);
  h->xb.end(nB);
  if (first) h->xa.hist = h->xb.hist = 0;
  for (size_t i = 0; i < h->res.size(); ++i) {
    const int nf = h->res[i].stage == 0 ? n : (h->res[i].stage == 1 ? nB : nD);
    h->n1[i].end(nf);
    h->n2[i].end(nf);
  }
  h->nout.end(nD);
}

void reset_rings(wan_vae* h) {
  h->pq.reset();
  h->xa.reset();
  h->xb.reset();
  h->nout.reset();
  for (Seq& q : h->n1) q.reset();
  for (Seq& q : h->n2) q.reset();
}

wan_status check_tensor(const wan_tensor* t, const char* what, int ndim) {
  VREQ(t, WAN_ERR_INVALID_ARG, "%s is NULL", what);
  VREQ(t->ndim == ndim, WAN_ERR_SHAPE, "%s: expected %d dimensions, got %d", what, ndim, t->ndim);
  VREQ(t->dtype == WAN_F32 || t->dtype == WAN_BF16, WAN_ERR_DTYPE, "%s: dtype must be WAN_F32 or WAN_BF16", what);
  for (int i = 0; i < ndim; ++i) VREQ(t->shape[i] >= 0, WAN_ERR_SHAPE, "%s: negative dimension", what);
  return WAN_OK;
}

}  // namespace

// =====================================================================================================
// C ABI
// =====================================================================================================

extern "C" const char* wan_vae_last_error(void) { return g_verr.c_str(); }

extern "C" int64_t wan_vae_device_bytes(const wan_vae* h) { return h ? (int64_t)(h->wbytes + h->abytes) : 0; }

extern "C" void wan_vae_destroy(wan_vae* h) { free_vae(h); }

extern "C" wan_status wan_vae_create(const wan_vae_config* cfg, const wan_weight* weights, size_t n_weights,
                                     void* hip_stream, wan_vae** out) {
  g_verr.clear();
  VREQ(out, WAN_ERR_INVALID_ARG, "out handle pointer is NULL");
  *out = nullptr;
  VREQ(cfg, WAN_ERR_INVALID_ARG, "config is NULL");
  VREQ(cfg->z_dim == 16, WAN_ERR_UNSUPPORTED, "z_dim must be 16 (got %d)", cfg->z_dim);
  VREQ(cfg->base_dim >= 1 && cfg->base_dim <= 256, WAN_ERR_UNSUPPORTED, "base_dim must be in [1, 256]");
  VREQ(cfg->chunk_frames >= 1 && cfg->chunk_frames <= 4, WAN_ERR_INVALID_ARG, "chunk_frames must be in [1, 4]");
  VREQ(cfg->eps > 0.0f && cfg->eps < 1.0f, WAN_ERR_INVALID_ARG, "eps must be in (0, 1)");
  VREQ(cfg->max_height >= 1 && cfg->max_width >= 1, WAN_ERR_INVALID_ARG, "max_height / max_width must be >= 1");
  VREQ(cfg->max_height <= 2048 && cfg->max_width <= 2048, WAN_ERR_UNSUPPORTED,
       "max_height / max_width above 2048 latent pixels");
  VREQ(weights || !n_weights, WAN_ERR_INVALID_ARG, "weights is NULL");

  wan_vae* h = new wan_vae();
  h->cfg = *cfg;
  (void)hipGetDevice(&h->device);
  build_layout(h);

  // ---- names and shapes
  const std::vector<Expect> exp = expected(h);
  std::unordered_map<std::string, size_t> by_name;
  for (size_t i = 0; i < n_weights; ++i) {
    const wan_weight& w = weights[i];
    if (!w.name) { free_vae(h); return vfail(WAN_ERR_INVALID_ARG, "weight %zu has no name", i); }
    if (!by_name.emplace(w.name, i).second) {
      free_vae(h);
      return vfail(WAN_ERR_MISSING_WEIGHT, "weight %s given twice", w.name);
    }
  }
  for (const Expect& e : exp) {
    auto it = by_name.find(e.name);
    if (it == by_name.end()) { free_vae(h); return vfail(WAN_ERR_MISSING_WEIGHT, "missing weight %s", e.name.c_str()); }
    const wan_weight& w = weights[it->second];
    if (w.dtype != WAN_F32 && w.dtype != WAN_BF16) {
      free_vae(h);
      return vfail(WAN_ERR_DTYPE, "weight %s: bad dtype", e.name.c_str());
    }
    bool ok = w.ndim == (int)e.shape.size();
    for (int d = 0; ok && d < w.ndim; ++d) ok = w.shape[d] == e.shape[d];
    if (!ok) {
      free_vae(h);
      return vfail(WAN_ERR_SHAPE, "weight %s has shape %s, expected %s", e.name.c_str(),
                   shape_str(w.shape, w.ndim).c_str(), shape_str(e.shape.data(), (int)e.shape.size()).c_str());
    }
    if (!w.data) { free_vae(h); return vfail(WAN_ERR_INVALID_ARG, "weight %s: data is NULL", e.name.c_str()); }
  }
  if (by_name.size() != exp.size()) {
    std::unordered_map<std::string, int> want;
    for (const Expect& e : exp) want[e.name] = 1;
    for (auto& kv : by_name)
      if (!want.count(kv.first)) {
        free_vae(h);
        return vfail(WAN_ERR_MISSING_WEIGHT, "unexpected weight %s", kv.first.c_str());
      }
  }

  // ---- allocate
  Arena pw, pa;
  plan_weights(h, pw);
  plan_acts(h, pa);
  h->wbytes = pw.used;
  h->abytes = pa.used;
  if (hipMalloc(&h->wmem, h->wbytes) != hipSuccess) {
    (void)hipGetLastError();
    free_vae(h);
    return vfail(WAN_ERR_OOM, "could not allocate %zu bytes of packed weights", pw.used);
  }
  if (hipMalloc(&h->amem, h->abytes) != hipSuccess) {
    (void)hipGetLastError();
    free_vae(h);
    return vfail(WAN_ERR_OOM, "could not allocate %zu bytes of frame buffers", pa.used);
  }
  Arena aw{(char*)h->wmem, 0}, aa{(char*)h->amem, 0};
  plan_weights(h, aw);
  plan_acts(h, aa);

  // ---- pack
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e = hipSuccess;
  auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
  auto W = [&](const std::string& n) -> const wan_weight& { return weights[by_name.at(n)]; };
  auto vec = [&](const std::string& n, float* dst) {
    const wan_weight& w = W(n);
    int64_t cnt = 1;
    for (int d = 0; d < w.ndim; ++d) cnt *= w.shape[d];
    chk(launch_pack_f32(w.data, w.dtype, cnt, dst, s));
  };
  auto conv = [&](const std::string& wn, const std::string& bn, const ConvW& c) {
    const wan_weight& w = W(wn);
    chk(launch_vae_pack_conv(w.data, w.dtype, c.cout, c.cin, c.kt, c.ks, c.ncf, c.w, s));
    vec(bn, c.b);
  };
  chk(launch_vae_zero(h->wmem, (int64_t)h->wbytes, s));       // padding of biases and gains
  chk(launch_vae_zero(h->amem, (int64_t)h->abytes, s));       // frame borders and the zero frame
  vec("latents_mean", h->mean);
  vec("latents_std", h->stdv);
  vec("post_quant_conv.weight", h->wq);
  vec("post_quant_conv.bias", h->bq);
  conv("decoder.conv_in.weight", "decoder.conv_in.bias", h->conv_in);
  for (const ResW& r : h->res) {
    vec(r.name + ".norm1.gamma", r.g1);
    vec(r.name + ".norm2.gamma", r.g2);
    conv(r.name + ".conv1.weight", r.name + ".conv1.bias", r.c1);
    conv(r.name + ".conv2.weight", r.name + ".conv2.bias", r.c2);
    if (r.has_sc) conv(r.name + ".conv_shortcut.weight", r.name + ".conv_shortcut.bias", r.sc);
  }
  for (const UpW& u : h->up) {
    if (u.time) conv(u.name + ".time_conv.weight", u.name + ".time_conv.bias", u.tc);
    conv(u.name + ".resample.1.weight", u.name + ".resample.1.bias", u.rs);
  }
  vec("decoder.norm_out.gamma", h->g_out);
  conv("decoder.conv_out.weight", "decoder.conv_out.bias", h->conv_out);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free_vae(h);
    return vfail(WAN_ERR_HIP, "weight packing failed: %s", hipGetErrorString(e));
  }
  *out = h;
  return WAN_OK;
}

extern "C" wan_status wan_vae_decode(wan_vae* h, const wan_tensor* latent, wan_tensor* video, void* hip_stream) {
  g_verr.clear();
  VREQ(h, WAN_ERR_INVALID_ARG, "handle is NULL");
  int dev = -1;
  VHIP(hipGetDevice(&dev), "hipGetDevice");
  VREQ(dev == h->device, WAN_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  wan_status st = check_tensor(latent, "latent", 5);
  if (st != WAN_OK) return st;
  st = check_tensor(video, "video", 5);
  if (st != WAN_OK) return st;
  const int64_t B = latent->shape[0], F = latent->shape[2], H = latent->shape[3], W = latent->shape[4];
  VREQ(latent->shape[1] == h->cfg.z_dim, WAN_ERR_SHAPE, "latent has %lld channels, expected %d",
       (long long)latent->shape[1], h->cfg.z_dim);
  VREQ(B == 0 || F >= 1, WAN_ERR_SHAPE, "latent needs at least one frame");
  VREQ(H >= 1 && W >= 1, WAN_ERR_SHAPE, "latent height and width must be >= 1");
  VREQ(H <= h->cfg.max_height && W <= h->cfg.max_width, WAN_ERR_SHAPE,
       "latent %lld x %lld exceeds the handle's max %lld x %lld", (long long)H, (long long)W,
       (long long)h->cfg.max_height, (long long)h->cfg.max_width);
  const int64_t T = B == 0 ? 0 : 1 + 4 * (F - 1);
  const int64_t want[5] = {B, 3, T, 8 * H, 8 * W};
  for (int d = 0; d < 5; ++d)
    VREQ(video->shape[d] == want[d], WAN_ERR_SHAPE, "video has shape %s, expected %s",
         shape_str(video->shape, 5).c_str(), shape_str(want, 5).c_str());
  if (B == 0) return WAN_OK;
  VREQ(latent->data && video->data, WAN_ERR_INVALID_ARG, "latent / video data is NULL");
  const int64_t zb = (latent->dtype == WAN_BF16 ? 2 : 4) * 16 * F * H * W;
  const int64_t vb = (video->dtype == WAN_BF16 ? 2 : 4) * 3 * T * 64 * H * W;
  const char *z0 = (const char*)latent->data, *v0 = (const char*)video->data;
  VREQ(z0 + B * zb <= v0 || v0 + B * vb <= z0, WAN_ERR_INVALID_ARG, "video must not overlap the latent");

  hipStream_t s = (hipStream_t)hip_stream;
  Ctx x{h, s};
  for (int st2 = 0; st2 < 4; ++st2) {
    x.H[st2] = H << st2;
    x.W[st2] = W << st2;
  }
  if (H != h->cur_h || W != h->cur_w) {
    // frame layouts change with the size: clear every frame buffer so that all borders are zero again
    VHIP(launch_vae_zero(h->amem, (int64_t)h->abytes, s), "clearing the frame buffers");
    h->cur_h = H;
    h->cur_w = W;
  }
  for (int64_t bi = 0; bi < B; ++bi) {
    reset_rings(h);
    const void* z = z0 + bi * zb;
    void* v = (char*)video->data + bi * vb;
    decode_chunk(x, z, latent->dtype, F, 0, 1, true, v, video->dtype, T, 0);
    for (int64_t f0 = 1; f0 < F; f0 += h->cfg.chunk_frames) {
      const int n = (int)(F - f0 < h->cfg.chunk_frames ? F - f0 : h->cfg.chunk_frames);
      decode_chunk(x, z, latent->dtype, F, f0, n, false, v, video->dtype, T, 1 + 4 * (f0 - 1));
    }
    if (x.err != hipSuccess) break;
  }
  VHIP(x.err, "decode launch");
  return WAN_OK;
}

extern "C" wan_status wan_vae_time_convs(wan_vae* h, int64_t max_launches) {
  g_verr.clear();
  VREQ(h, WAN_ERR_INVALID_ARG, "handle is NULL");
  VREQ(max_launches >= 0 && max_launches <= (1 << 20), WAN_ERR_INVALID_ARG, "max_launches out of range");
  int dev = -1;
  VHIP(hipGetDevice(&dev), "hipGetDevice");
  VREQ(dev == h->device, WAN_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  release_events(h);
  for (int64_t i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      (void)hipGetLastError();
      release_events(h);
      return vfail(WAN_ERR_HIP, "hipEventCreate failed");
    }
    h->ev.push_back(e);
  }
  return WAN_OK;
}

extern "C" wan_status wan_vae_conv_time(wan_vae* h, double* total_ms, int64_t* launches, double* flops) {
  g_verr.clear();
  VREQ(h && total_ms && launches && flops, WAN_ERR_INVALID_ARG, "NULL argument");
  int dev = -1;
  VHIP(hipGetDevice(&dev), "hipGetDevice");
  VREQ(dev == h->device, WAN_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  double sum = 0.0;
  for (int64_t i = 0; i + 1 < h->ev_used; i += 2) {
    VHIP(hipEventSynchronize(h->ev[i + 1]), "hipEventSynchronize");
    float ms = 0.0f;
    VHIP(hipEventElapsedTime(&ms, h->ev[i], h->ev[i + 1]), "hipEventElapsedTime");
    sum += ms;
  }
  *total_ms = sum;
  *launches = h->ev_used / 2;
  *flops = h->ev_flops;
  h->ev_used = 0;
  h->ev_flops = 0.0;
  return WAN_OK;
}

// ---- per-stage entry points ---------------------------------------------------------------------------

extern "C" int64_t wan_vae_op_packed_conv_elems(int64_t c_out, int64_t c_in, int32_t kt, int32_t ks) {
  if (c_out <= 0 || c_in <= 0 || (kt != 1 && kt != 3) || (ks != 1 && ks != 3)) return -1;
  return vae_packed_conv_elems(c_out, c_in, kt, ks, ncf_for(c_out));
}

extern "C" wan_status wan_vae_op_pack_conv(const void* w, int32_t dtype, int64_t c_out, int64_t c_in, int32_t kt,
                                           int32_t ks, void* dst, void* hip_stream) {
  g_verr.clear();
  VREQ(w && dst, WAN_ERR_INVALID_ARG, "pack_conv: NULL pointer");
  VREQ(dtype == WAN_F32 || dtype == WAN_BF16, WAN_ERR_DTYPE, "pack_conv: bad dtype");
  VREQ(c_out > 0 && c_in > 0 && (kt == 1 || kt == 3) && (ks == 1 || ks == 3), WAN_ERR_SHAPE,
       "pack_conv: c_out, c_in > 0, kt and ks in {1, 3}");
  VHIP(launch_vae_pack_conv(w, dtype, c_out, c_in, kt, ks, ncf_for(c_out), (bf16_t*)dst, (hipStream_t)hip_stream),
       "pack_conv");
  return WAN_OK;
}

extern "C" wan_status wan_vae_op_conv(const void* const* in, int32_t kt, int32_t ks, int32_t up, const void* w_packed,
                                      const float* bias, int64_t c_in, int64_t c_out, int32_t split, int64_t H,
                                      int64_t W, void* const* out, const void* const* res, int32_t nf, void* hip_stream) {
  g_verr.clear();
  VREQ(in && out && w_packed && bias, WAN_ERR_INVALID_ARG, "conv: NULL pointer");
  VREQ(nf >= 1 && nf <= VAE_MAXF, WAN_ERR_INVALID_ARG, "conv: nf must be in [1, %d]", VAE_MAXF);
  VREQ(kt == 1 || kt == 3, WAN_ERR_INVALID_ARG, "conv: kt must be 1 or 3");
  VREQ(ks == 1 || ks == 3, WAN_ERR_INVALID_ARG, "conv: ks must be 1 or 3");
  VREQ(up == 0 || (up == 1 && kt == 1 && ks == 3), WAN_ERR_INVALID_ARG, "conv: up needs kt = 1 and ks = 3");
  VREQ(split == 1 || split == 2, WAN_ERR_INVALID_ARG, "conv: split must be 1 or 2");
  VREQ(!(split == 2 && (ks != 1 || kt != 3)), WAN_ERR_UNSUPPORTED, "conv: split = 2 is the (3,1,1) time conv");
  VREQ(c_in > 0 && c_in % 16 == 0, WAN_ERR_SHAPE, "conv: c_in must be a positive multiple of 16");
  VREQ(c_out > 0 && (split == 1 ? (c_out % 16 == 0 || c_out < 16) : (c_out % 32 == 0)), WAN_ERR_SHAPE,
       "conv: c_out must be a multiple of 16 (or < 16), and of 32 with split = 2");
  VREQ(H >= 1 && W >= 1 && H <= 16384 && W <= 16384, WAN_ERR_SHAPE, "conv: H, W must be in [1, 16384]");
  VREQ(!up || (H % 2 == 0 && W % 2 == 0), WAN_ERR_SHAPE, "conv: up needs even H and W");
  for (int i = 0; i < nf * kt; ++i) VREQ(in[i], WAN_ERR_INVALID_ARG, "conv: in[%d] is NULL (pass a zero frame)", i);
  for (int i = 0; i < nf * split; ++i) VREQ(out[i], WAN_ERR_INVALID_ARG, "conv: out[%d] is NULL", i);
  ConvW c;
  c.w = (bf16_t*)w_packed;
  c.cin = c_in;
  c.cout = c_out;
  c.kt = kt;
  c.ks = ks;
  c.ncf = ncf_for(c_out);
  // the kernel reads 32 * ncf bias values per tile: stage a padded copy when c_out is not a whole tile
  VREQ(c_out % (32 * c.ncf) == 0, WAN_ERR_UNSUPPORTED,
       "conv: c_out must be a multiple of 32 (96 for the wide tiles) in the stand-alone op");
  c.b = (float*)bias;
  VaeConvArgs a{};
  for (int j = 0; j < nf; ++j)
    for (int dt = 0; dt < kt; ++dt) a.in[j][dt] = (const bf16_t*)in[j * kt + dt];
  for (int i = 0; i < nf * split; ++i) {
    a.out[i] = (bf16_t*)out[i];
    a.res[i] = res ? (const bf16_t*)res[i] : nullptr;
  }
  Ctx x{nullptr, (hipStream_t)hip_stream};
  x.H[0] = H;
  x.W[0] = W;
  conv_launch(x, c, a, 0, nf, up, split, false);
  VHIP(x.err, "conv");
  return WAN_OK;
}

extern "C" wan_status wan_vae_op_rms_silu(const void* const* in, void* const* out, int32_t nf, int64_t c, int64_t H,
                                          int64_t W, const float* gamma, float eps, void* hip_stream) {
  g_verr.clear();
  VREQ(in && out && gamma, WAN_ERR_INVALID_ARG, "rms_silu: NULL pointer");
  VREQ(nf >= 1 && nf <= VAE_MAXF, WAN_ERR_INVALID_ARG, "rms_silu: nf must be in [1, %d]", VAE_MAXF);
  VREQ(c >= 1 && c <= 4096, WAN_ERR_SHAPE, "rms_silu: c must be in [1, 4096]");
  VREQ(H >= 1 && W >= 1, WAN_ERR_SHAPE, "rms_silu: H, W must be >= 1");
  VREQ(eps > 0.0f, WAN_ERR_INVALID_ARG, "rms_silu: eps must be > 0");
  for (int j = 0; j < nf; ++j) VREQ(in[j] && out[j] && in[j] != out[j], WAN_ERR_INVALID_ARG, "rms_silu: frame %d", j);
  VREQ(c % 16 == 0, WAN_ERR_UNSUPPORTED, "rms_silu: the stand-alone op needs c a multiple of 16");
  VHIP(launch_vae_rms_silu((const bf16_t* const*)in, (bf16_t* const*)out, nf, c, c / 16, H, W, gamma, eps,
                           (hipStream_t)hip_stream),
       "rms_silu");
  return WAN_OK;
}
