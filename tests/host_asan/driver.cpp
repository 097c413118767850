// Host-only sanitizer run of the library's C ABI (test infrastructure; built by tests/test_host_asan.py
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code, the HIP runtime replaced by
// hip_stub.cpp, so every kernel launch is checked for its launch shape and skipped).
//
// usage: driver SPEC_FILE
// The spec file, written by the test from the seeded workload definitions, lists configurations and
// their weights:
//   DIT <tag> <field>=<value> ...        a wan_dit_config (fields by name)
//   VAE <tag> <field>=<value> ...        a wan_vae_config
//   W <name> <dtype> <ndim> <d0> ...     a weight of the configuration above it
// Every call's status is checked against the expected one; the run ends with "ALL OK" and exit code 0.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <sstream>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "wan_dit.h"
#include "wan_ops.h"
#include "wan_vae.h"

extern "C" long stub_launches();
extern "C" long stub_bad_launches();
extern "C" long stub_live_allocs();

namespace {

int g_fail = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d (%s | %s)\n", what, got, want, wan_dit_last_error(),
                 wan_vae_last_error());
    ++g_fail;
  }
}

struct Spec {
  std::string kind, tag;
  std::map<std::string, double> f;
  struct W {
    std::string name;
    int dtype;
    std::vector<int64_t> shape;
  };
  std::vector<W> w;
};

std::vector<Spec> read_spec(const char* path) {
  std::ifstream in(path);
  std::vector<Spec> out;
  std::string line;
  while (std::getline(in, line)) {
    std::istringstream ss(line);
    std::string k;
    ss >> k;
    if (k == "DIT" || k == "VAE") {
      Spec s;
      s.kind = k;
      ss >> s.tag;
      std::string kv;
      while (ss >> kv) {
        const size_t e = kv.find('=');
        s.f[kv.substr(0, e)] = std::atof(kv.c_str() + e + 1);
      }
      out.push_back(s);
    } else if (k == "W") {
      Spec::W w;
      int nd = 0;
      ss >> w.name >> w.dtype >> nd;
      for (int i = 0; i < nd; ++i) {
        int64_t d;
        ss >> d;
        w.shape.push_back(d);
      }
      out.back().w.push_back(w);
    }
  }
  return out;
}

// device (here: host) buffers for a weight list, as wan_weight entries
struct Weights {
  std::vector<wan_weight> list;
  std::vector<void*> mem;
  explicit Weights(const Spec& s) {
    for (const auto& w : s.w) {
      int64_t n = 1;
      for (int64_t d : w.shape) n *= d;
      void* p = nullptr;
      hipMalloc(&p, (size_t)n * (w.dtype == WAN_BF16 ? 2 : 4));
      mem.push_back(p);
      wan_weight e{};
      e.name = w.name.c_str();
      e.data = p;
      e.dtype = w.dtype;
      e.ndim = (int)w.shape.size();
      for (size_t i = 0; i < w.shape.size(); ++i) e.shape[i] = w.shape[i];
      list.push_back(e);
    }
  }
  ~Weights() {
    for (void* p : mem) hipFree(p);
  }
};

struct Tensor {
  wan_tensor t{};
  explicit Tensor(std::vector<int64_t> shape, int dtype = WAN_F32) {
    int64_t n = 1;
    for (int64_t d : shape) n *= d;
    hipMalloc(&t.data, (size_t)(n > 0 ? n : 1) * (dtype == WAN_BF16 ? 2 : 4));
    t.dtype = dtype;
    t.ndim = (int)shape.size();
    for (size_t i = 0; i < shape.size(); ++i) t.shape[i] = shape[i];
  }
  ~Tensor() { hipFree(t.data); }
  Tensor(const Tensor&) = delete;
};

wan_dit_config dit_config(const Spec& s) {
  wan_dit_config c{};
  auto g = [&](const char* k) { return s.f.at(k); };
  c.dim = (int)g("dim"); c.num_heads = (int)g("num_heads"); c.head_dim = (int)g("head_dim");
  c.ffn_dim = (int)g("ffn_dim"); c.num_layers = (int)g("num_layers"); c.in_channels = (int)g("in_channels");
  c.out_channels = (int)g("out_channels"); c.text_dim = (int)g("text_dim"); c.freq_dim = (int)g("freq_dim");
  c.patch_t = 1; c.patch_h = 2; c.patch_w = 2;
  c.rope_dim_t = (int)g("rope_dim_t"); c.rope_dim_h = (int)g("rope_dim_h"); c.rope_dim_w = (int)g("rope_dim_w");
  c.per_token_timestep = (int)g("per_token_timestep"); c.eps = 1e-6f; c.rope_theta = 1e4;
  c.max_batch = (int64_t)g("max_batch"); c.max_tokens = (int64_t)g("max_tokens");
  c.max_text_len = (int64_t)g("max_text_len"); c.max_image_len = (int64_t)g("max_image_len");
  c.image_dim = (int)g("image_dim");
  return c;
}

void run_dit(const Spec& s) {
  const wan_dit_config cfg = dit_config(s);
  Weights w(s);
  wan_dit* h = nullptr;
  // create failures first: a missing, a duplicate, a mis-shaped and a mis-typed weight
  {
    std::vector<wan_weight> l = w.list;
    l.pop_back();
    expect(wan_dit_create(&cfg, l.data(), l.size(), nullptr, &h), WAN_ERR_MISSING_WEIGHT, "dit missing weight");
    l = w.list;
    l.push_back(l[0]);
    expect(wan_dit_create(&cfg, l.data(), l.size(), nullptr, &h), WAN_ERR_MISSING_WEIGHT, "dit duplicate weight");
    l = w.list;
    l[1].shape[0] += 1;
    expect(wan_dit_create(&cfg, l.data(), l.size(), nullptr, &h), WAN_ERR_SHAPE, "dit weight shape");
    l = w.list;
    l[2].dtype = 7;
    expect(wan_dit_create(&cfg, l.data(), l.size(), nullptr, &h), WAN_ERR_DTYPE, "dit weight dtype");
  }
  expect(wan_dit_create(&cfg, w.list.data(), w.list.size(), nullptr, &h), WAN_OK, "dit create");
  if (!h) return;
  const int64_t B = cfg.max_batch, C = cfg.in_channels, F = (int64_t)s.f.at("frames");
  const int64_t Hz = (int64_t)s.f.at("height"), Wz = (int64_t)s.f.at("width"), Lt = cfg.max_text_len;
  const int64_t L = F * (Hz / 2) * (Wz / 2);
  Tensor lat({B, C, F, Hz, Wz}), t({B}), txt({B, Lt, cfg.text_dim}), out({B, cfg.out_channels, F, Hz, Wz});
  expect(wan_dit_forward(h, &lat.t, &t.t, &txt.t, &out.t, nullptr), WAN_OK, "dit forward");
  Tensor tt({B, L});
  expect(wan_dit_forward(h, &lat.t, &tt.t, &txt.t, &out.t, nullptr),
         cfg.per_token_timestep ? WAN_OK : WAN_ERR_UNSUPPORTED, "dit forward per-token t");
  Tensor bad({B, C, F, Hz + 1, Wz});
  expect(wan_dit_forward(h, &bad.t, &t.t, &txt.t, &out.t, nullptr), WAN_ERR_SHAPE, "dit forward odd height");
  Tensor big({B + 1, C, F, Hz, Wz}), tb({B + 1}), xb({B + 1, Lt, cfg.text_dim}), ob({B + 1, cfg.out_channels, F, Hz, Wz});
  expect(wan_dit_forward(h, &big.t, &tb.t, &xb.t, &ob.t, nullptr), WAN_ERR_SHAPE, "dit forward batch > max");
  expect(wan_dit_forward(h, &lat.t, &t.t, nullptr, &out.t, nullptr), WAN_ERR_INVALID_ARG, "dit forward null text");
  if (cfg.max_image_len > 0) {
    Tensor img({B, cfg.max_image_len, cfg.image_dim});
    expect(wan_dit_forward_image(h, &lat.t, &t.t, &txt.t, &img.t, &out.t, nullptr), WAN_OK, "dit forward image");
  }
  if (B >= 2) {
    Tensor l1({1, C, F, Hz, Wz}), t1({1}), pair({2, Lt, cfg.text_dim}), xn({1, cfg.out_channels, F, Hz, Wz});
    expect(wan_dit_denoise_step(h, &l1.t, &t1.t, &pair.t, nullptr, 6.0f, 0.75f, 0.5f, &xn.t, nullptr), WAN_OK,
           "dit denoise step");
    expect(wan_dit_denoise_step(h, &l1.t, &t1.t, &pair.t, nullptr, 6.0f, 0.75f, 0.5f, &l1.t, nullptr),
           WAN_ERR_INVALID_ARG, "dit denoise step aliasing");
  }
  expect(wan_dit_time_attention(h, 8), WAN_OK, "dit time attention");
  expect(wan_dit_forward(h, &lat.t, &t.t, &txt.t, &out.t, nullptr), WAN_OK, "dit timed forward");
  double ms = 0;
  int64_t n = 0;
  expect(wan_dit_attention_time(h, &ms, &n), WAN_OK, "dit attention time");
  if (n != cfg.num_layers) {
    std::fprintf(stderr, "FAIL timed launches %lld, expected %d\n", (long long)n, cfg.num_layers);
    ++g_fail;
  }
  expect(wan_dit_time_attention(h, 0), WAN_OK, "dit timing off");
  wan_dit_destroy(h);
}

void run_vae(const Spec& s) {
  wan_vae_config c{};
  c.z_dim = 16;
  c.base_dim = (int)s.f.at("base_dim");
  c.chunk_frames = (int)s.f.at("chunk_frames");
  c.eps = 1e-6f;
  c.max_height = (int64_t)s.f.at("max_height");
  c.max_width = (int64_t)s.f.at("max_width");
  Weights w(s);
  wan_vae* h = nullptr;
  {
    std::vector<wan_weight> l = w.list;
    l.erase(l.begin() + 5);
    expect(wan_vae_create(&c, l.data(), l.size(), nullptr, &h), WAN_ERR_MISSING_WEIGHT, "vae missing weight");
    l = w.list;
    l[4].shape[1] += 16;   // decoder.conv_in.weight [4b, 16, 3, 3, 3]: wrong input channels
    expect(wan_vae_create(&c, l.data(), l.size(), nullptr, &h), WAN_ERR_SHAPE, "vae weight shape");
  }
  expect(wan_vae_create(&c, w.list.data(), w.list.size(), nullptr, &h), WAN_OK, "vae create");
  if (!h) return;
  const int64_t H = c.max_height, W = c.max_width;
  for (int64_t F : {1, 2, 6, 9}) {
    Tensor z({2, 16, F, H, W}, WAN_BF16), v({2, 3, 1 + 4 * (F - 1), 8 * H, 8 * W});
    expect(wan_vae_decode(h, &z.t, &v.t, nullptr), WAN_OK, "vae decode");
  }
  {
    Tensor z({1, 16, 5, H - 1, W - 2}), v({1, 3, 17, 8 * (H - 1), 8 * (W - 2)}, WAN_BF16);
    expect(wan_vae_decode(h, &z.t, &v.t, nullptr), WAN_OK, "vae decode smaller");
    Tensor vbad({1, 3, 16, 8 * (H - 1), 8 * (W - 2)});
    expect(wan_vae_decode(h, &z.t, &vbad.t, nullptr), WAN_ERR_SHAPE, "vae decode frames");
    Tensor zbig({1, 16, 2, H + 1, W}), vbig({1, 3, 5, 8 * (H + 1), 8 * W});
    expect(wan_vae_decode(h, &zbig.t, &vbig.t, nullptr), WAN_ERR_SHAPE, "vae decode too tall");
    expect(wan_vae_decode(h, &z.t, &z.t, nullptr), WAN_ERR_SHAPE, "vae decode video = latent");
  }
  expect(wan_vae_time_convs(h, 64), WAN_OK, "vae time convs");
  {
    Tensor z({1, 16, 3, H, W}), v({1, 3, 9, 8 * H, 8 * W});
    expect(wan_vae_decode(h, &z.t, &v.t, nullptr), WAN_OK, "vae timed decode");
  }
  double ms = 0, fl = 0;
  int64_t n = 0;
  expect(wan_vae_conv_time(h, &ms, &n, &fl), WAN_OK, "vae conv time");
  expect(wan_vae_time_convs(h, 0), WAN_OK, "vae timing off");
  wan_vae_destroy(h);
}

void run_ops() {
  // the allocation-free attention: its static workspace (here the host shadow of the device array)
  const int64_t B = 1, L = 300, nh = 2, D = 128 * nh, ldv = 320;
  Tensor q({B * L, 3 * D}, WAN_BF16), vt({B, nh, 128, ldv}, WAN_BF16), o({B * L, D}, WAN_BF16);
  expect(wan_op_attention_noalloc(q.t.data, 3 * D, (char*)q.t.data + 2 * D, 3 * D, vt.t.data, ldv, o.t.data, D, B, L, L,
                                  (int)nh, nullptr),
         WAN_OK, "attention noalloc");
  expect(wan_op_attention_noalloc(q.t.data, 3 * D, (char*)q.t.data + 2 * D, 3 * D, vt.t.data, ldv, o.t.data, D, 4200,
                                  L, L, (int)nh, nullptr),
         WAN_ERR_UNSUPPORTED, "attention noalloc too large");
  // GEMM with a workspace: 36 x 17 tiles of 256, 100 in the last round -> the stream-K chunks and fix-up
  {
    const int64_t M = 9000, N = 4104, K = 256;
    Tensor x({M, K}, WAN_BF16), w({N, K}, WAN_BF16), bias({N}), ob({M, N}, WAN_BF16), of({M, N}), tab({N}),
        src({(M + 99) / 100, N});
    const int64_t wsb = wan_op_gemm_workspace_bytes();
    Tensor ws({wsb / 4});
    for (int epi = 0; epi <= 4; ++epi) {
      void* out = epi < 2 ? ob.t.data : of.t.data;
      expect(wan_op_gemm_ws(x.t.data, K, w.t.data, K, (const float*)bias.t.data, M, N, K, epi, out, N,
                            (const float*)tab.t.data, (const float*)src.t.data, N, 100, ws.t.data, wsb, nullptr),
             WAN_OK, "gemm_ws");
    }
    expect(wan_op_gemm_ws(x.t.data, K, w.t.data, K, (const float*)bias.t.data, M, N, K, 0, ob.t.data, N, nullptr,
                          nullptr, 0, 1, ws.t.data, wsb - 16, nullptr),
           WAN_ERR_INVALID_ARG, "gemm_ws short workspace");
    expect(wan_op_gemm_ws(x.t.data, K, w.t.data, K, (const float*)bias.t.data, M, N, K, 0, ob.t.data, N, nullptr,
                          nullptr, 0, 1, (char*)ws.t.data + 4, wsb - 16, nullptr),
           WAN_ERR_INVALID_ARG, "gemm_ws misaligned workspace");
    expect(wan_op_gemm_ws(x.t.data, K, w.t.data, K, (const float*)bias.t.data, M, N, 100, 0, ob.t.data, N, nullptr,
                          nullptr, 0, 1, ws.t.data, wsb, nullptr),
           WAN_ERR_SHAPE, "gemm_ws K not a multiple of 64");
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: driver SPEC_FILE\n");
    return 2;
  }
  const std::vector<Spec> specs = read_spec(argv[1]);
  for (const Spec& s : specs) {
    std::printf("case %s %s (%zu weights)\n", s.kind.c_str(), s.tag.c_str(), s.w.size());
    if (s.kind == "DIT") run_dit(s);
    else run_vae(s);
  }
  run_ops();
  std::printf("launches %ld, bad launch shapes %ld, live allocations %ld\n", stub_launches(), stub_bad_launches(),
              stub_live_allocs());
  if (stub_bad_launches() != 0 || stub_live_allocs() != 0) ++g_fail;
  if (g_fail) {
    std::printf("FAILED %d\n", g_fail);
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
