// Host side of the MI355X Wan2.2 TI2V-5B VAE decoder: the C ABI of include/wanvae.h,
// argument validation (done before anything is launched), topology inference from the
// parameter shapes, the workspace plan, the chunk loop that enqueues the kernels (two
// stages per chunk, pipelined over two streams), and the spatially tiled decode.
//
// What is computed follows FastVideo's "wan22_vae_decode reference.py" page: post_quant_conv
// over all latent frames, then one latent frame per chunk through conv_in, the mid block
// (residual block, attention, residual block), up blocks 0-3, norm_out + SiLU and conv_out,
// the chunks' frames written straight into the video (unpatchified and clamped).
//
// Causal caches ("Causal caches" section): every conv with a 3-frame kernel owns a ring
// of frames in the workspace. The producer of the conv's input (a norm pass or a conv
// epilogue) writes the chunk's frames into the ring's next slots; the conv reads its last
// <= 2 frames (history) and the new ones through a frame-pointer table, zeros standing in
// for missing history. No cache is ever copied or concatenated.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "internal.h"
#include "wanvae.h"

namespace wanvae {

static thread_local std::string g_err;

static int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int report(int code, const char* msg) {
  g_err = msg;
  return code;
}

#define HIP_TRY(expr)                                                                         \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(WANVAE_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

static size_t esize(int dtype) { return dtype == kBF16 ? 2 : 4; }

// ------------------------------------------------------------------ kernel timing

struct ProfRec {
  hipEvent_t a, b;
  int kind;
  double flops, bytes;
};

struct Profiler {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t event() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void clear() {
    for (auto& r : recs) {
      pool.push_back(r.a);
      pool.push_back(r.b);
    }
    recs.clear();
  }
};

static thread_local Profiler g_prof;

// Starts timing a launch on st (a no-op unless timing is enabled).
static hipEvent_t prof_start(hipStream_t st) {
  if (!g_prof.on) return nullptr;
  hipEvent_t a = g_prof.event();
  if (a && hipEventRecord(a, st) != hipSuccess) return nullptr;
  return a;
}

static void prof_stop(hipEvent_t a, int kind, double flops, double bytes, hipStream_t st) {
  if (!a) return;
  hipEvent_t b = g_prof.event();
  if (!b || hipEventRecord(b, st) != hipSuccess) return;
  g_prof.recs.push_back({a, b, kind, flops, bytes});
}
static int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------------ workspace planning

// Bump allocator: with base == nullptr it only measures.
struct Arena {
  char* base = nullptr;
  size_t used = 0;
  void* take(size_t bytes) {
    size_t off = align_up((int64_t)used, 256);
    used = off + align_up((int64_t)bytes, 256);
    return base ? base + off : nullptr;
  }
};

// A frame table: n frames, each [B][H][W][C] at f[i] (nullptr = zero frame), batch stride bs elements.
struct FrameRef {
  void* f[kMaxFrames] = {};
  int64_t bs[kMaxFrames] = {};
  int n = 0;
  void push(void* p, int64_t s) {
    f[n] = p;
    bs[n++] = s;
  }
};

static FrameRef frames_of(void* base, int F, int64_t frame_elems, int64_t bs, size_t es) {
  FrameRef r;
  for (int t = 0; t < F; ++t) r.push(base ? (char*)base + (int64_t)t * frame_elems * es : nullptr, bs);
  return r;
}

// Ring of frames holding a causal conv's input: history and the current chunk.
struct Ring {
  char* base = nullptr;
  int64_t fbytes = 0, bs = 0;
  int R = 0, head = 0, count = 0;
  void* slot(int k) const { return base + (int64_t)(((k % R) + R) % R) * fbytes; }
  FrameRef write(int F) const {
    FrameRef r;
    for (int t = 0; t < F; ++t) r.push(slot(head + t), bs);
    return r;
  }
  // the conv's time-padded input: 2 - hist zero frames, hist history frames, F new frames
  FrameRef read(int F) const {
    FrameRef r;
    const int hist = std::min(count, 2);
    for (int z = 0; z < 2 - hist; ++z) r.push(nullptr, bs);
    for (int k = 0; k < hist; ++k) r.push(slot(head - hist + k), bs);
    for (int t = 0; t < F; ++t) r.push(slot(head + t), bs);
    return r;
  }
  void commit(int F) {
    head = (head + F) % R;
    count += F;
  }
};

// ------------------------------------------------------------------ parameters and topology

struct ConvSpec {
  std::string name;
  int Cout, Cin, kt, kh, kw;
  bool conv2d;  // [Co, Ci, kh, kw]
};

struct Topology {
  int base = 0, c4 = 0, c2 = 0, c1 = 0, z = 48;
  std::vector<ConvSpec> convs;
  std::vector<std::pair<std::string, int>> norms;  // gamma name, C
};

struct UpSpec {
  int cin, cout;
  bool temporal, spatial;
};

static void up_specs(int base, UpSpec u[4]) {
  u[0] = {4 * base, 4 * base, true, true};
  u[1] = {4 * base, 4 * base, true, true};
  u[2] = {4 * base, 2 * base, false, true};
  u[3] = {2 * base, base, false, false};
}

static void make_topology(int base, Topology& tp) {
  tp.base = base;
  tp.c4 = 4 * base;
  tp.c2 = 2 * base;
  tp.c1 = base;
  auto conv = [&](const std::string& n, int co, int ci, int kt, int kh, int kw, bool c2d = false) {
    tp.convs.push_back({n, co, ci, kt, kh, kw, c2d});
  };
  auto resnet = [&](const std::string& p, int ci, int co) {
    tp.norms.push_back({p + ".norm1.gamma", ci});
    conv(p + ".conv1", co, ci, 3, 3, 3);
    tp.norms.push_back({p + ".norm2.gamma", co});
    conv(p + ".conv2", co, co, 3, 3, 3);
    if (ci != co) conv(p + ".conv_shortcut", co, ci, 1, 1, 1);
  };
  const int c = tp.c4;
  conv("post_quant_conv", tp.z, tp.z, 1, 1, 1);
  conv("decoder.conv_in", c, tp.z, 3, 3, 3);
  resnet("decoder.mid_block.resnets.0", c, c);
  tp.norms.push_back({"decoder.mid_block.attentions.0.norm.gamma", c});
  conv("decoder.mid_block.attentions.0.to_qkv", 3 * c, c, 1, 1, 1, true);
  conv("decoder.mid_block.attentions.0.proj", c, c, 1, 1, 1, true);
  resnet("decoder.mid_block.resnets.1", c, c);
  UpSpec u[4];
  up_specs(base, u);
  for (int i = 0; i < 4; ++i) {
    const std::string p = "decoder.up_blocks." + std::to_string(i);
    for (int j = 0; j < 3; ++j) resnet(p + ".resnets." + std::to_string(j), j == 0 ? u[i].cin : u[i].cout, u[i].cout);
    if (u[i].temporal) conv(p + ".upsampler.time_conv", 2 * u[i].cout, u[i].cout, 3, 1, 1);
    if (u[i].spatial) conv(p + ".upsampler.resample.1", u[i].cout, u[i].cout, 1, 3, 3, true);
  }
  tp.norms.push_back({"decoder.norm_out.gamma", base});
  conv("decoder.conv_out", 12, base, 3, 3, 3);
}

using WeightMap = std::unordered_map<std::string, const wanvae_tensor*>;

static bool has_prefix(const char* s, const char* p) { return strncmp(s, p, strlen(p)) == 0; }

static int64_t numel(const wanvae_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

static int check_tensor(const wanvae_tensor* t, const char* what) {
  if (!t) return fail(WANVAE_EARG, "%s: NULL tensor", what);
  if (t->dtype != kF32 && t->dtype != kBF16)
    return fail(WANVAE_EDTYPE, "%s: element type %d is neither WANVAE_F32 nor WANVAE_BF16", what, t->dtype);
  if (t->ndim < 0 || t->ndim > 5) return fail(WANVAE_ESHAPE, "%s: ndim %d not in [0, 5]", what, t->ndim);
  if (!t->data) return fail(WANVAE_EARG, "%s: NULL data pointer", what);
  for (int i = 0; i < t->ndim; ++i)
    if (t->shape[i] < 0) return fail(WANVAE_ESHAPE, "%s: negative extent", what);
  return WANVAE_OK;
}

static int parse_weights(const wanvae_tensor* ws, int64_t n, WeightMap& m) {
  if (n < 0 || (n > 0 && !ws)) return fail(WANVAE_EARG, "weights: NULL table or negative count");
  for (int64_t i = 0; i < n; ++i) {
    const wanvae_tensor* t = ws + i;
    if (!t->name) return fail(WANVAE_EARG, "weights[%lld]: NULL name", (long long)i);
    if (!has_prefix(t->name, "decoder.") && !has_prefix(t->name, "post_quant_conv.")) continue;
    if (!m.emplace(t->name, t).second) return fail(WANVAE_EARG, "duplicate parameter name %s", t->name);
    if (int rc = check_tensor(t, t->name)) return rc;
  }
  return WANVAE_OK;
}

static bool shape_is(const wanvae_tensor* t, std::initializer_list<int64_t> s) {
  if (t->ndim != (int)s.size()) return false;
  int i = 0;
  for (int64_t v : s)
    if (t->shape[i++] != v) return false;
  return true;
}

static std::string shape_str(const wanvae_tensor* t) {
  std::string s = "[";
  for (int i = 0; i < t->ndim; ++i) s += (i ? "," : "") + std::to_string(t->shape[i]);
  return s + "]";
}

static int build_topology(const WeightMap& m, Topology& tp) {
  auto it = m.find("decoder.conv_out.weight");
  if (it == m.end()) return fail(WANVAE_EMISSING, "missing parameter decoder.conv_out.weight");
  if (it->second->ndim != 5) return fail(WANVAE_ESHAPE, "decoder.conv_out.weight: shape %s", shape_str(it->second).c_str());
  const int64_t base = it->second->shape[1];
  auto pq = m.find("post_quant_conv.weight");
  if (pq == m.end()) return fail(WANVAE_EMISSING, "missing parameter post_quant_conv.weight");
  if (pq->second->ndim != 5 || pq->second->shape[0] != 48)
    return fail(WANVAE_ETOPOLOGY, "post_quant_conv.weight %s: the decoder needs z_dim 48", shape_str(pq->second).c_str());
  // the widths run on every kernel the decoder launches: the mid-block attention needs
  // 4 * base in {64, 128, 256, 384, 512, 1024}
  if (base < 16 || base % 16 != 0 || 4 * base > 1024 || !attn_supported(4 * (int)base, kBF16))
    return fail(WANVAE_ETOPOLOGY, "decoder_base_dim %lld unsupported (16, 32, 64, 96, 128 or 256)", (long long)base);
  make_topology((int)base, tp);
  for (const ConvSpec& c : tp.convs) {
    const std::string wn = c.name + ".weight", bn = c.name + ".bias";
    auto w = m.find(wn);
    if (w == m.end()) return fail(WANVAE_EMISSING, "missing parameter %s", wn.c_str());
    auto b = m.find(bn);
    if (b == m.end()) return fail(WANVAE_EMISSING, "missing parameter %s", bn.c_str());
    bool ok;
    if (c.conv2d)
      ok = shape_is(w->second, {c.Cout, c.Cin, c.kh, c.kw}) ||
           (c.kh == 1 && shape_is(w->second, {c.Cout, c.Cin}));
    else
      ok = shape_is(w->second, {c.Cout, c.Cin, c.kt, c.kh, c.kw});
    if (!ok) return fail(WANVAE_ESHAPE, "%s: shape %s does not fit the decoder", wn.c_str(), shape_str(w->second).c_str());
    if (!shape_is(b->second, {c.Cout}))
      return fail(WANVAE_ESHAPE, "%s: shape %s, expected [%d]", bn.c_str(), shape_str(b->second).c_str(), c.Cout);
  }
  for (auto& g : tp.norms) {
    auto w = m.find(g.first);
    if (w == m.end()) return fail(WANVAE_EMISSING, "missing parameter %s", g.first.c_str());
    if (numel(w->second) != g.second)
      return fail(WANVAE_ESHAPE, "%s: %lld elements, expected %d", g.first.c_str(), (long long)numel(w->second), g.second);
  }
  return WANVAE_OK;
}

// ------------------------------------------------------------------ launch helpers

struct ConvW {
  void* w = nullptr;
  float* b = nullptr;
  int Cout = 0, Cin = 0, kt = 1, kh = 1, kw = 1;
};

static int prep_conv(Arena& ar, int dtype, const wanvae_tensor* w, const wanvae_tensor* b, int Cout, int Cin, int kt,
                     int kh, int kw, ConvW& out, hipStream_t st) {
  out.Cout = Cout, out.Cin = Cin, out.kt = kt, out.kh = kh, out.kw = kw;
  const int taps = kt * kh * kw;
  out.w = ar.take((size_t)Cout * taps * Cin * esize(dtype));
  out.b = (float*)ar.take((size_t)Cout * 4);
  if (!ar.base) return WANVAE_OK;
  hipEvent_t e0 = prof_start(st);
  HIP_TRY(launch_repack(w->data, w->dtype, out.w, dtype, Cout, Cin, taps, st));
  HIP_TRY(launch_to_f32(b->data, b->dtype, out.b, Cout, dtype, st));
  prof_stop(e0, WANVAE_KOTHER, 0, (double)Cout * taps * Cin * (esize(w->dtype) + esize(dtype)), st);
  return WANVAE_OK;
}

static int prep_vec(Arena& ar, int dtype, const wanvae_tensor* g, int C, float*& out, hipStream_t st) {
  out = (float*)ar.take((size_t)C * 4);
  if (!ar.base) return WANVAE_OK;
  HIP_TRY(launch_to_f32(g->data, g->dtype, out, C, dtype, st));
  return WANVAE_OK;
}

// Tile of the conv kernel for a layer. WANVAE_CONV_TILE (a ConvTile value) overrides the
// choice for the bf16 layers with more than 64 output channels, for tuning.
static std::atomic<int> g_conv_kernel{[] {
  const char* e = getenv("WANVAE_CONV_TILE");
  const int k = e ? atoi(e) : -1;
  return k >= -1 && k < WANVAE_CONV_KERNELS ? k : -1;
}()};

// The bf16 norm's SiLU: -1 automatic (the LDS table on large launches), 0 arithmetic only,
// 1 the table on every launch. WANVAE_NORM_TAB gives the initial setting.
static std::atomic<int> g_norm_kernel{[] {
  const char* e = getenv("WANVAE_NORM_TAB");
  const int k = e ? atoi(e) : -1;
  return k >= -1 && k <= 1 ? k : -1;
}()};

static int pick_tile(const ConvArgs& a, int dtype) {
  const int forced = g_conv_kernel.load(std::memory_order_relaxed);
  const int Cout = a.Cout;
  const int64_t M = (int64_t)a.F * a.B * a.Ho * a.Wo;
  // bf16: the direct-to-LDS kernels (Cout % 8 == 0 for the frame / interleave / q-k-v stores;
  // the unpatchify + clamp store of conv_out on the 16-channel tile)
  if (dtype == kBF16 && a.mode == kEpiVideo && Cout <= 16 && Cout % 4 == 0) {
    // conv_out: the 16-channel halo tile on frames of at least 32 x 64
    const bool halo16 = conv_halo_supported(a, dtype, kTileHalo16x16x32);
    if (forced == kTileHalo16x16x32 && halo16) return forced;
    if (forced == kTileDma16x256) return forced;
    return halo16 && a.Ho >= 32 && a.Wo >= 64 ? kTileHalo16x16x32 : kTileDma16x256;
  }
  const bool dma_ok = a.mode != kEpiVideo && Cout % 8 == 0 && Cout > 64;
  if (!dma_ok) return Cout <= 64 ? kTile32x256 : kTile128x128;
  if (dtype != kBF16) {
    // fp32 on the direct-to-LDS tiles (no halo kernel, no split K): 128 x 256 with two
    // workgroups per CU (faster on every decoder shape than the 256 x 256 tiles, whose
    // fp32 fragments leave one wave per SIMD), 128 x 128 for the small level-0 frames
    if (forced >= kTileDma256x128 && forced <= kTileDma256x256w8b) return forced;
    return M < 16384 ? kTileDma128x128 : kTileDma128x256;
  }
  const bool halo = conv_halo_supported(a, dtype, kTileHalo128x16x32);
  const bool forced_halo = forced == kTileHalo128x16x32 || forced == kTileHalo128x16x16 || forced == kTileHalo128x32x16;
  if (forced >= 0 && forced != kTileHalo16x16x32 && (!forced_halo || halo)) return forced;
  // 3x3 convs on frames of at least 32 x 64: the halo tile (input patch shared by the nine
  // spatial taps), 16 x 32 blocks, or 16 x 16 blocks with split K where the frames leave
  // the chip short of blocks (the level-0 layers: 3,520 positions per frame); 256 x 256
  // tiles (8 waves of 64 x 128) for the other convs with enough positions to fill the chip;
  // 128 x 128 (with split K) for the rest
  if (halo && a.Ho >= 32 && a.Wo >= 64) {
    if (M < 16384) return kTileHalo128x16x16;
    // 512-position blocks in the orientation that pads the frame less (16 x 32 on a tie):
    // 32 x 16 for the 320 x 176 frames of a portrait video's level 2
    auto up = [](int64_t v, int64_t m) { return (v + m - 1) / m * m; };
    return up(a.Ho, 32) * up(a.Wo, 16) < up(a.Ho, 16) * up(a.Wo, 32) ? kTileHalo128x32x16 : kTileHalo128x16x32;
  }
  if (M < 16384) return kTileDma128x128;
  return Cout % 256 == 0 ? kTileDma256x256w8b : kTileDma256x128;
}

// Scratch for the float32 partial sums of split-K convs, set by the entry point for the
// duration of a call (thread-local: calls are synchronous on their host thread).
struct SplitBuf {
  float* p = nullptr;
  size_t floats = 0;
};
static thread_local SplitBuf t_split;
struct SplitScope {
  SplitBuf prev;
  explicit SplitScope(SplitBuf b) : prev(t_split) { t_split = b; }
  ~SplitScope() { t_split = prev; }
};

// Partial-sum floats to reserve for convs over M positions with up to Cout channels: convs
// with fewer than 16,384 positions (the 128 x 128 tile) split K up to 4 ways.
static size_t split_floats(int64_t M, int64_t Cout) { return M < 16384 ? (size_t)4 * M * Cout : 0; }

static SplitBuf take_split(Arena& ar, int64_t M, int64_t Cout) {
  SplitBuf b;
  b.floats = split_floats(M, Cout);
  if (b.floats) b.p = (float*)ar.take(b.floats * 4);
  return b;
}

// Compute units of the current device (256 on an MI355X), looked up once per process.
static int64_t cu_count() {
  static const int64_t n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return (int64_t)v;
  }();
  return n;
}

// K split of a direct-to-LDS conv: enough workgroups for about three per CU when the tiles
// alone leave the chip short, at least 16 K steps per range, within the partials scratch. The
// halo tile (one workgroup per CU) takes the split that its time estimate favours.
static int split_for(const ConvArgs& a, int tile, int dtype, const SplitBuf& sb) {
  int TC = 0, TP = 0, TPY = 0, TPX = 0;
  switch (tile) {
    case kTileDma256x128: TC = 256, TP = 128; break;
    case kTileDma256x256: case kTileDma256x256w8: case kTileDma256x256w8b: TC = 256, TP = 256; break;
    case kTileDma128x128: TC = 128, TP = 128; break;
    case kTileDma128x256: TC = 128, TP = 256; break;
    case kTileDma16x256: TC = 16, TP = 256; break;
    case kTileHalo128x16x32: TC = 128, TPY = 16, TPX = 32; break;
    case kTileHalo128x16x16: TC = 128, TPY = 16, TPX = 16; break;
    case kTileHalo128x32x16: TC = 128, TPY = 32, TPX = 16; break;
    default: return 1;
  }
  if (dtype != kBF16 || a.mode == kEpiVideo || a.Cout % 8 || sb.p == nullptr) return 1;
  const int64_t M = (int64_t)a.F * a.B * a.Ho * a.Wo;
  const int64_t nct = (a.Cout + TC - 1) / TC;
  // tiles, and the K units a range must hold: 16 steps of 32 channels, or (halo tile) 4 groups
  // of nine taps
  int64_t tiles, units;
  if (TPX) {
    tiles = nct * ((a.Ho + TPY - 1) / TPY) * ((a.Wo + TPX - 1) / TPX) * a.F * a.B;
    units = a.kt * (a.Cin / 32) / 4;
  } else {
    tiles = nct * ((M + TP - 1) / TP);
    units = a.kt * a.kh * a.kw * ((a.Cin + 31) / 32) / 16;
  }
  if (tiles >= 512) return 1;
  int ks;
  if (TPX) {
    // halo tile, one workgroup per CU: the split with the least estimated time, rounds of
    // workgroups over the CUs x (the range's steps + the tile's fixed cost, about 16.5 us:
    // 46 steps of a 16 x 16 block, 23 of a 512-position block)
    const int64_t steps = (int64_t)a.kt * 9 * (a.Cin / 32), fixed = TPX * TPY == 256 ? 46 : 23;
    const int64_t ncu = cu_count();
    int64_t best = -1;
    ks = 1;
    for (int k = 1; k <= std::min<int64_t>(4, std::max<int64_t>(units, 1)); ++k) {
      if ((size_t)k * M * a.Cout > sb.floats) break;
      const int64_t t = (tiles * k + ncu - 1) / ncu * (steps / k + fixed);
      if (best < 0 || t < best) best = t, ks = k;
    }
    return ks;
  }
  ks = (int)std::min<int64_t>({4, (768 + tiles - 1) / tiles, units});
  while (ks > 1 && (size_t)ks * M * a.Cout > sb.floats) --ks;
  return std::max(ks, 1);
}

struct ConvCall {
  ConvArgs a;
  ConvCall() { memset(&a, 0, sizeof a); }
};

static int run_conv(const ConvW& cw, const FrameRef& in, int B, int Hin, int Win, int Ho, int Wo, int F, bool up,
                    ConvCall& cc, int dtype, hipStream_t st) {
  ConvArgs& a = cc.a;
  if (in.n != F + cw.kt - 1 || in.n > kMaxFrames)
    return fail(WANVAE_EARG, "internal: conv frame table has %d frames for %d outputs", in.n, F);
  for (int i = 0; i < in.n; ++i) {
    a.in[i] = in.f[i];
    a.in_bs[i] = in.bs[i];
  }
  a.B = B, a.Hin = Hin, a.Win = Win, a.Cin = cw.Cin;
  a.Ho = Ho, a.Wo = Wo, a.Cout = cw.Cout;
  a.kt = cw.kt, a.kh = cw.kh, a.kw = cw.kw;
  a.up = up ? 1 : 0;
  a.F = F;
  a.w = cw.w;
  a.bias = cw.b;
  const int tile = pick_tile(a, dtype);
  a.ksplit = split_for(a, tile, dtype, t_split);
  a.part = t_split.p;
  // algorithmic FLOPs: every output, every spatial tap, the time taps on real frames
  double taps_real = 0;
  for (int t = 0; t < F; ++t)
    for (int dt = 0; dt < cw.kt; ++dt) taps_real += in.f[t + dt] ? 1 : 0;
  const double flops = 2.0 * B * Ho * Wo * (double)cw.Cout * cw.Cin * cw.kh * cw.kw * taps_real;
  hipEvent_t e0 = prof_start(st);
  HIP_TRY(launch_conv(a, dtype, tile, st));
  prof_stop(e0, WANVAE_KCONV, flops, 0, st);
  return WANVAE_OK;
}

static void set_out(ConvArgs& a, const FrameRef& o, int outC) {
  for (int i = 0; i < o.n; ++i) {
    a.out[i] = o.f[i];
    a.out_bs[i] = o.bs[i];
  }
  a.outC = outC;
}

static void set_res(ConvArgs& a, const FrameRef& r) {
  a.has_res = 1;
  for (int i = 0; i < r.n; ++i) {
    a.res[i] = r.f[i];
    a.res_bs[i] = r.bs[i];
  }
}

static int run_norm(const FrameRef& in, const FrameRef& out, int F, int B, int HW, int C, const float* gamma, bool silu,
                    int dtype, hipStream_t st) {
  NormArgs n;
  memset(&n, 0, sizeof n);
  if (in.n < F || out.n < F) return fail(WANVAE_EARG, "internal: norm frame tables too short");
  for (int t = 0; t < F; ++t) {
    n.in[t] = in.f[t];
    n.in_bs[t] = in.bs[t];
    n.out[t] = out.f[t];
    n.out_bs[t] = out.bs[t];
  }
  n.F = F, n.B = B, n.HW = HW, n.C = C;
  n.gamma = gamma;
  n.sqrtC = (float)std::sqrt((double)C);
  n.silu = silu ? 1 : 0;
  n.tab = g_norm_kernel.load(std::memory_order_relaxed);
  hipEvent_t e0 = prof_start(st);
  HIP_TRY(launch_norm(n, dtype, st));
  prof_stop(e0, WANVAE_KNORM, 0, 2.0 * F * B * (double)HW * C * esize(dtype), st);
  return WANVAE_OK;
}

// Attention block on nfr independent frames folded into the batch (F = 1, B = nfr):
// n = RMS norm (no SiLU) -> 1x1 conv to q, k, v^T -> attention core -> 1x1 proj + x. The
// bf16 core runs on the materialised-score kernels (k_attn_mm: scores GEMM with the tile
// softmax, per-tile weights, P V GEMM); fp32 (and bf16 with WANVAE_ATTN_FLASH=1, for
// comparison) on the flash kernel.
struct AttnBufs {
  void *n = nullptr, *q = nullptr, *k = nullptr, *vt = nullptr, *o = nullptr;
  int S = 0, Sp = 0;
  SplitBuf split;  // the standalone block's split-K scratch (the decoder has its own)
  int ksplit = 1;  // attention key ranges, and their partial results
  float* opart = nullptr;
  float* ml = nullptr;
  bool mm = false;  // materialised scores: P, each key tile's (max, sum) and weight per query
  void* p = nullptr;
  float2* tml = nullptr;
  float* fac = nullptr;
  int nkt = 0;
};

static const bool g_attn_flash = [] {
  const char* e = getenv("WANVAE_ATTN_FLASH");
  return e && atoi(e) != 0;
}();

// Attention key ranges: with fewer than 256 workgroups of 32 queries, up to 4 ranges of keys
// run as separate workgroups (the frames of one chunk would leave most of the chip idle).
static int attn_split(int nfr, int S) {
  const int64_t qtiles = (int64_t)nfr * ((S + 31) / 32);
  if (qtiles >= 256) return 1;
  return (int)std::min<int64_t>({4, (512 + qtiles - 1) / qtiles, (S + 31) / 32});
}

static void plan_attn_bufs(Arena& ar, AttnBufs& ab, int nfr, int S, int C, int dtype, bool with_split) {
  const size_t es = esize(dtype);
  ab.S = S;
  ab.Sp = (int)align_up(S, 32);
  ab.n = ar.take((size_t)nfr * S * C * es);
  ab.q = ar.take((size_t)nfr * S * C * es);
  ab.k = ar.take((size_t)nfr * S * C * es);
  ab.vt = ar.take((size_t)nfr * C * ab.Sp * es);
  ab.o = ar.take((size_t)nfr * S * C * es);
  if (with_split) ab.split = take_split(ar, (int64_t)nfr * S, 3 * (int64_t)C);
  ab.mm = dtype == kBF16 && !g_attn_flash;
  if (ab.mm) {
    ab.nkt = (S + 127) / 128;
    ab.p = ar.take((size_t)nfr * S * ab.Sp * es);
    ab.tml = (float2*)ar.take((size_t)nfr * ab.nkt * S * sizeof(float2));
    ab.fac = (float*)ar.take((size_t)nfr * ab.nkt * S * sizeof(float));
    ab.ksplit = 1;
    return;
  }
  ab.ksplit = attn_split(nfr, S);
  if (ab.ksplit > 1) {
    ab.opart = (float*)ar.take((size_t)ab.ksplit * nfr * S * C * 4);
    ab.ml = (float*)ar.take((size_t)ab.ksplit * nfr * S * 2 * 4);
  }
}

static int run_attn(const FrameRef& x, const FrameRef& y, int nfr, int H, int W, int C, const float* gamma,
                    const ConvW& qkv, const ConvW& proj, const AttnBufs& ab, int dtype, hipStream_t st) {
  const size_t es = esize(dtype);
  const int S = H * W;
  const FrameRef n = frames_of(ab.n, 1, (int64_t)nfr * S * C, (int64_t)S * C, es);
  if (int rc = run_norm(x, n, 1, nfr, S, C, gamma, false, dtype, st)) return rc;
  HIP_TRY(hipMemsetAsync(ab.vt, 0, (size_t)nfr * C * ab.Sp * es, st));
  {
    ConvCall cc;
    cc.a.mode = kEpiQKV;
    cc.a.outC = C;
    cc.a.q = ab.q, cc.a.k = ab.k, cc.a.vt = ab.vt;
    cc.a.S = S, cc.a.Sp = ab.Sp;
    if (int rc = run_conv(qkv, n, nfr, H, W, H, W, 1, false, cc, dtype, st)) return rc;
  }
  hipEvent_t e0 = prof_start(st);
  if (ab.mm) {
    AttnMatArgs am;
    am.q = ab.q, am.k = ab.k, am.vt = ab.vt, am.o = ab.o;
    am.p = ab.p, am.ml = ab.tml, am.fac = ab.fac;
    am.nfr = nfr, am.S = S, am.Sp = ab.Sp, am.C = C, am.nkt = ab.nkt;
    am.sc = (float)(1.4426950408889634 / std::sqrt((double)C));
    HIP_TRY(launch_attn_mm(am, st));
  } else {
    AttnArgs aa;
    aa.q = ab.q, aa.k = ab.k, aa.vt = ab.vt, aa.o = ab.o;
    aa.nfr = nfr, aa.S = S, aa.Sp = ab.Sp, aa.C = C;
    aa.scale = (float)(1.0 / std::sqrt((double)C));
    aa.ksplit = ab.ksplit, aa.opart = ab.opart, aa.ml = ab.ml;
    HIP_TRY(launch_attn(aa, dtype, st));
  }
  prof_stop(e0, WANVAE_KATTN, 4.0 * nfr * (double)S * S * C, 0, st);
  {
    ConvCall cc;
    cc.a.mode = kEpiFrames;
    set_out(cc.a, y, C);
    set_res(cc.a, x);
    const FrameRef o = frames_of(ab.o, 1, (int64_t)nfr * S * C, (int64_t)S * C, es);
    if (int rc = run_conv(proj, o, nfr, H, W, H, W, 1, false, cc, dtype, st)) return rc;
  }
  return WANVAE_OK;
}

// ------------------------------------------------------------------ the decoder

struct Level {
  int H = 0, W = 0, F = 0, C = 0;  // resolution, max frames per chunk, max channels
  void* x[3] = {};
  void* h = nullptr;
  void* s = nullptr;
  void* tb = nullptr;  // time conv output (2F frames), up blocks 0 and 1
};

// Streams and events of the two-stage chunk pipeline of the decoder: one set per device,
// made on first use and kept until the process ends. Both streams have the default priority
// and do not synchronise with the null stream; the events carry no timing.
struct Pipe {
  std::mutex mu;  // held while one decode enqueues its work on these streams
  hipStream_t s[2] = {};
  hipEvent_t start = nullptr, end[2] = {}, a[2] = {}, b[2] = {};
};
static std::atomic<int> g_pipeline{1};

static int pipe_for_device(Pipe** out) {
  static std::mutex mu;
  static std::map<int, std::unique_ptr<Pipe>> pipes;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(mu);
  std::unique_ptr<Pipe>& slot = pipes[dev];
  if (!slot) {
    std::unique_ptr<Pipe> p(new Pipe);
    for (int k = 0; k < 2; ++k) HIP_TRY(hipStreamCreateWithFlags(&p->s[k], hipStreamNonBlocking));
    hipEvent_t* ev[7] = {&p->start, &p->end[0], &p->end[1], &p->a[0], &p->a[1], &p->b[0], &p->b[1]};
    for (hipEvent_t* e : ev) HIP_TRY(hipEventCreateWithFlags(e, hipEventDisableTiming));
    slot = std::move(p);
  }
  *out = slot.get();
  return WANVAE_OK;
}

class Decoder {
 public:
  Decoder(const WeightMap& m, const Topology& tp, int dtype, int B, int T, int h, int w)
      : m_(m), tp_(tp), dt_(dtype), es_(esize(dtype)), B_(B), T_(T), h_(h), w_(w) {}

  // Lays out the workspace (measuring when ar.base is null) and, with a real base, enqueues
  // the weight preparation.
  int plan(Arena& ar, hipStream_t st) {
    if (int rc = plan_weights(ar, st)) return rc;
    return plan_acts(ar);
  }

  // The weights in the compute type and the kernels' layout (enqueued on st with a real base).
  int plan_weights(Arena& ar, hipStream_t st) {
    st_ = st;
    for (const ConvSpec& c : tp_.convs) {
      ConvW& cw = cw_[c.name];
      if (int rc = prep_conv(ar, dt_, m_.at(c.name + ".weight"), m_.at(c.name + ".bias"), c.Cout, c.Cin, c.kt, c.kh,
                             c.kw, cw, st))
        return rc;
    }
    for (auto& g : tp_.norms)
      if (int rc = prep_vec(ar, dt_, m_.at(g.first), g.second, gam_[g.first], st)) return rc;
    return WANVAE_OK;
  }

  // Runs on the weights another decoder of the same parameters prepared.
  void use_weights(const Decoder& o, hipStream_t st) {
    cw_ = o.cw_;
    gam_ = o.gam_;
    st_ = st;
  }

  // Activations, caches and scratch.
  int plan_acts(Arena& ar) {
    const int c4 = tp_.c4, c2 = tp_.c2, c1 = tp_.c1;
    up_specs(tp_.base, u_);
    const int fmax[4] = {1, T_ > 1 ? 2 : 1, T_ > 1 ? 4 : 1, T_ > 1 ? 4 : 1};
    const int cmax[4] = {c4, c4, c4, c2};
    for (int l = 0; l < 4; ++l) {
      Level& L = lv_[l];
      L.H = h_ << l, L.W = w_ << l, L.F = fmax[l], L.C = cmax[l];
      const size_t bytes = (size_t)L.F * B_ * L.H * L.W * L.C * es_;
      for (int i = 0; i < 3; ++i) L.x[i] = ar.take(bytes);
      L.h = ar.take(bytes);
      if (l >= 2) L.s = ar.take(bytes);
      if (l <= 1) L.tb = ar.take(2 * bytes);
    }
    zt_ = ar.take((size_t)T_ * B_ * h_ * w_ * tp_.z * es_);
    pq_ = ar.take((size_t)T_ * B_ * h_ * w_ * tp_.z * es_);
    // rings of the 3-frame convs: conv1/conv2 of every residual block, the time convs, conv_out
    auto ring = [&](const std::string& name, int l, int C) {
      Ring& r = rings_[name];
      const Level& L = lv_[l];
      r.R = L.F + 2;
      r.fbytes = (int64_t)B_ * L.H * L.W * C * es_;
      r.bs = (int64_t)L.H * L.W * C;
      r.base = (char*)ar.take((size_t)r.R * r.fbytes);
    };
    auto resnet_rings = [&](const std::string& p, int l, int ci, int co) {
      ring(p + ".conv1", l, ci);
      ring(p + ".conv2", l, co);
    };
    resnet_rings("decoder.mid_block.resnets.0", 0, c4, c4);
    resnet_rings("decoder.mid_block.resnets.1", 0, c4, c4);
    const UpSpec* u = u_;
    for (int i = 0; i < 4; ++i) {
      const std::string p = "decoder.up_blocks." + std::to_string(i);
      for (int j = 0; j < 3; ++j) resnet_rings(p + ".resnets." + std::to_string(j), i, j == 0 ? u[i].cin : u[i].cout, u[i].cout);
      if (u[i].temporal) ring(p + ".upsampler.time_conv", i, u[i].cout);
    }
    ring("decoder.conv_out", 3, c1);
    plan_attn_bufs(ar, ab_, B_, h_ * w_, c4, dt_, false);
    // level 1's input frames, second buffer (odd chunks)
    x1b_ = ar.take((size_t)lv_[1].F * B_ * lv_[1].H * lv_[1].W * lv_[1].C * es_);
    // split-K scratch for the level-0 convs (one frame of B x h x w positions; at most 3 c4
    // output channels, the attention's q-k-v conv), one per stage so that the two stages can
    // run at once with the same split of every conv
    splitA_ = take_split(ar, (int64_t)B_ * h_ * w_, 3 * (int64_t)c4);
    splitB_ = take_split(ar, (int64_t)B_ * h_ * w_, 3 * (int64_t)c4);
    return WANVAE_OK;
  }

  // Enqueues the decode. With `pipe`, chunk i's first stage (conv_in, the mid block and up
  // block 0, on pipe->s[0]) runs while chunk i-1's second stage (up blocks 1-3 and conv_out,
  // on pipe->s[1]) is still running; every kernel gets the arguments it gets without `pipe`.
  int run(const void* z, int z_dtype, void* video, Pipe* pipe) {
    {
      SplitScope scope(splitA_);
      HIP_TRY(launch_ncthw_to_frames(z, z_dtype, zt_, dt_, B_, tp_.z, tp_.z, T_, h_, w_, st_));
      // post_quant_conv over all T latent frames at once (frames folded into the batch)
      ConvCall cc;
      cc.a.mode = kEpiFrames;
      set_out(cc.a, frames_of(pq_, 1, 0, (int64_t)h_ * w_ * tp_.z, es_), tp_.z);
      const FrameRef in = frames_of(zt_, 1, 0, (int64_t)h_ * w_ * tp_.z, es_);
      if (int rc = run_conv(cw_.at("post_quant_conv"), in, T_ * B_, h_, w_, h_, w_, 1, false, cc, dt_, st_)) return rc;
    }
    if (!pipe) {
      for (int i = 0; i < T_; ++i) {
        {
          SplitScope scope(splitA_);
          if (int rc = chunk_a(i)) return rc;
        }
        SplitScope scope(splitB_);
        if (int rc = chunk_b(i, video)) return rc;
      }
      return WANVAE_OK;
    }
    const hipStream_t caller = st_;
    HIP_TRY(hipEventRecord(pipe->start, caller));
    for (int k = 0; k < 2; ++k) HIP_TRY(hipStreamWaitEvent(pipe->s[k], pipe->start, 0));
    int rc = WANVAE_OK;
    for (int i = 0; i < T_ && rc == WANVAE_OK; ++i) rc = pipelined_chunk(i, video, *pipe);
    st_ = caller;
    // the caller's stream waits for both stages, also after an error (the workspace may be
    // released on it next)
    for (int k = 0; k < 2; ++k) {
      hipError_t e = hipEventRecord(pipe->end[k], pipe->s[k]);
      if (e == hipSuccess) e = hipStreamWaitEvent(caller, pipe->end[k], 0);
      if (e != hipSuccess && rc == WANVAE_OK) rc = fail(WANVAE_EHIP, "joining the decode streams: %s", hipGetErrorString(e));
    }
    return rc;
  }

 private:
  FrameRef lvl_frames(int l, void* base, int F, int C) const {
    const Level& L = lv_[l];
    return frames_of(base, F, (int64_t)B_ * L.H * L.W * C, (int64_t)L.H * L.W * C, es_);
  }

  int conv_into(const std::string& name, const FrameRef& in, int l, int F, const FrameRef& out,
                const FrameRef* res) {
    const ConvW& cw = cw_.at(name);
    const Level& L = lv_[l];
    ConvCall cc;
    cc.a.mode = kEpiFrames;
    set_out(cc.a, out, cw.Cout);
    if (res) set_res(cc.a, *res);
    return run_conv(cw, in, B_, L.H, L.W, L.H, L.W, F, false, cc, dt_, st_);
  }

  // WanResidualBlock: x2 + shortcut with x1 = conv1(SiLU(norm1(x))), x2 = conv2(SiLU(norm2(x1)))
  int resnet(const std::string& p, int l, int F, const FrameRef& x, int ci, int co, const FrameRef& out) {
    const Level& L = lv_[l];
    const int HW = L.H * L.W;
    FrameRef res = x;
    if (ci != co) {
      res = lvl_frames(l, L.s, F, co);
      if (int rc = conv_into(p + ".conv_shortcut", x, l, F, res, nullptr)) return rc;
    }
    Ring& r1 = rings_.at(p + ".conv1");
    if (int rc = run_norm(x, r1.write(F), F, B_, HW, ci, gam_.at(p + ".norm1.gamma"), true, dt_, st_)) return rc;
    const FrameRef hbuf = lvl_frames(l, L.h, F, co);
    if (int rc = conv_into(p + ".conv1", r1.read(F), l, F, hbuf, nullptr)) return rc;
    r1.commit(F);
    Ring& r2 = rings_.at(p + ".conv2");
    if (int rc = run_norm(hbuf, r2.write(F), F, B_, HW, co, gam_.at(p + ".norm2.gamma"), true, dt_, st_)) return rc;
    if (int rc = conv_into(p + ".conv2", r2.read(F), l, F, out, &res)) return rc;
    r2.commit(F);
    return WANVAE_OK;
  }

  // Chunk i on the two pipeline streams. Level 1's input is double-buffered by chunk parity:
  // chunk i's first stage writes the buffer chunk i-2's second stage read, so it waits for
  // that stage; the second stage waits for its own chunk's first stage.
  int pipelined_chunk(int i, void* video, Pipe& pp) {
    const int par = i & 1;
    if (i >= 2) HIP_TRY(hipStreamWaitEvent(pp.s[0], pp.b[par], 0));
    st_ = pp.s[0];
    {
      SplitScope scope(splitA_);
      if (int rc = chunk_a(i)) return rc;
    }
    HIP_TRY(hipEventRecord(pp.a[par], pp.s[0]));
    HIP_TRY(hipStreamWaitEvent(pp.s[1], pp.a[par], 0));
    st_ = pp.s[1];
    {
      SplitScope scope(splitB_);
      if (int rc = chunk_b(i, video)) return rc;
    }
    HIP_TRY(hipEventRecord(pp.b[par], pp.s[1]));
    return WANVAE_OK;
  }

  // Input frames of up block b for chunk i (level 1: one buffer per chunk parity).
  void* block_in(int b, int i) const { return b == 1 && (i & 1) ? x1b_ : lv_[b].x[0]; }

  // Frames per chunk at level l: one for the first chunk (no time conv runs on it), else
  // doubled by each temporal up block below l.
  int frames_at(int l, int i) const {
    int F = 1;
    for (int b = 0; b < l && i > 0; ++b) F *= u_[b].temporal ? 2 : 1;
    return F;
  }

  // First stage of chunk i: conv_in, the mid block and up block 0.
  int chunk_a(int i) {
    const int c4 = tp_.c4;
    // conv_in: latent frames i-2, i-1 (history) and i, read in place from the post_quant output
    {
      FrameRef in;
      const int64_t fe = (int64_t)B_ * h_ * w_ * tp_.z;
      for (int s = i - 2; s <= i; ++s) in.push(s < 0 ? nullptr : (char*)pq_ + s * fe * es_, (int64_t)h_ * w_ * tp_.z);
      if (int rc = conv_into("decoder.conv_in", in, 0, 1, lvl_frames(0, lv_[0].x[0], 1, c4), nullptr)) return rc;
    }
    Level& L0 = lv_[0];
    const FrameRef x0 = lvl_frames(0, L0.x[0], 1, c4), x1 = lvl_frames(0, L0.x[1], 1, c4),
                   x2 = lvl_frames(0, L0.x[2], 1, c4);
    if (int rc = resnet("decoder.mid_block.resnets.0", 0, 1, x0, c4, c4, x1)) return rc;
    {
      const std::string a = "decoder.mid_block.attentions.0";
      if (int rc = run_attn(x1, x2, B_, h_, w_, c4, gam_.at(a + ".norm.gamma"), cw_.at(a + ".to_qkv"),
                            cw_.at(a + ".proj"), ab_, dt_, st_))
        return rc;
    }
    if (int rc = resnet("decoder.mid_block.resnets.1", 0, 1, x2, c4, c4, x0)) return rc;
    return up_block(0, i, nullptr);
  }

  // Second stage of chunk i: up blocks 1-3, norm_out, conv_out.
  int chunk_b(int i, void* video) {
    for (int b = 1; b < 4; ++b)
      if (int rc = up_block(b, i, video)) return rc;
    return WANVAE_OK;
  }

  // Up block b of chunk i: three residual blocks, then the upsampler into level b+1, or (the
  // last block) norm_out + SiLU and conv_out into the video.
  int up_block(int b, int i, void* video) {
    const bool first = i == 0;
    const UpSpec* u = u_;
    const int F = frames_at(b, i);
    Level& L = lv_[b];
    const std::string p = "decoder.up_blocks." + std::to_string(b);
    const FrameRef xin = lvl_frames(b, block_in(b, i), F, u[b].cin);
    const FrameRef xa = lvl_frames(b, L.x[1], F, u[b].cout), xb = lvl_frames(b, L.x[2], F, u[b].cout);
    if (int rc = resnet(p + ".resnets.0", b, F, xin, u[b].cin, u[b].cout, xa)) return rc;
    if (int rc = resnet(p + ".resnets.1", b, F, xa, u[b].cout, u[b].cout, xb)) return rc;
    const bool tconv = u[b].temporal && !first;
    Ring* tr = tconv ? &rings_.at(p + ".upsampler.time_conv") : nullptr;
    const FrameRef r2out = tconv ? tr->write(F) : xa;
    if (int rc = resnet(p + ".resnets.2", b, F, xb, u[b].cout, u[b].cout, r2out)) return rc;
    if (!u[b].spatial) {
      // norm_out + SiLU -> conv_out -> unpatchify + clamp straight into the video
      Ring& ro = rings_.at("decoder.conv_out");
      if (int rc = run_norm(r2out, ro.write(F), F, B_, L.H * L.W, u[b].cout, gam_.at("decoder.norm_out.gamma"), true,
                            dt_, st_))
        return rc;
      const ConvW& cw = cw_.at("decoder.conv_out");
      ConvCall cc;
      cc.a.mode = kEpiVideo;
      cc.a.video = video;
      cc.a.vF = 4 * T_ - 3;
      cc.a.vf0 = first ? 0 : 4 * i - 3;
      if (int rc = run_conv(cw, ro.read(F), B_, L.H, L.W, L.H, L.W, F, false, cc, dt_, st_)) return rc;
      ro.commit(F);
      return WANVAE_OK;
    }
    FrameRef src = r2out;
    int Fs = F;
    if (tconv) {
      // upsample3d's time conv: C -> 2C, channel c -> frame 2t, channel C + c -> frame 2t + 1
      const ConvW& cw = cw_.at(p + ".upsampler.time_conv");
      ConvCall cc;
      cc.a.mode = kEpiInterleave;
      src = lvl_frames(b, L.tb, 2 * F, u[b].cout);
      set_out(cc.a, src, u[b].cout);
      if (int rc = run_conv(cw, tr->read(F), B_, L.H, L.W, L.H, L.W, F, false, cc, dt_, st_)) return rc;
      tr->commit(F);
      Fs = 2 * F;
    }
    // upsample2d (nearest x2 read through the conv's addressing, 3x3 conv) + DupUp3D(block input)
    Level& N = lv_[b + 1];
    const ConvW& cw = cw_.at(p + ".upsampler.resample.1");
    ConvCall cc;
    cc.a.mode = kEpiFrames;
    set_out(cc.a, lvl_frames(b + 1, block_in(b + 1, i), Fs, u[b].cout), u[b].cout);
    const int ft = u[b].temporal ? 2 : 1;
    cc.a.has_dup = 1;
    for (int t = 0; t < F; ++t) {
      cc.a.dup[t] = xin.f[t];
      cc.a.dup_bs[t] = xin.bs[t];
    }
    cc.a.dup_C = u[b].cin;
    cc.a.dup_ft = ft;
    cc.a.dup_r = u[b].cout * ft * 4 / u[b].cin;
    cc.a.dup_shift = first ? ft - 1 : 0;
    return run_conv(cw, src, B_, L.H, L.W, N.H, N.W, Fs, true, cc, dt_, st_);
  }

  const WeightMap& m_;
  const Topology& tp_;
  int dt_;
  size_t es_;
  int B_, T_, h_, w_;
  hipStream_t st_ = nullptr;
  std::unordered_map<std::string, ConvW> cw_;
  std::unordered_map<std::string, float*> gam_;
  std::unordered_map<std::string, Ring> rings_;
  Level lv_[4];
  void* zt_ = nullptr;
  void* pq_ = nullptr;
  AttnBufs ab_;
  UpSpec u_[4];
  void* x1b_ = nullptr;
  SplitBuf splitA_, splitB_;
};

static int check_dtype(int dtype, const char* what) {
  if (dtype != kF32 && dtype != kBF16)
    return fail(WANVAE_EDTYPE, "%s must be WANVAE_F32 or WANVAE_BF16, not %d", what, dtype);
  return WANVAE_OK;
}

static int decode_validate(int64_t B, int64_t T, int64_t h, int64_t w, const wanvae_tensor* weights, int64_t n,
                           int32_t dtype, WeightMap& m, Topology& tp) {
  if (int rc = check_dtype(dtype, "dtype")) return rc;
  if (B < 1 || T < 1 || h < 1 || w < 1)
    return fail(WANVAE_ESHAPE, "latent shape [%lld, 48, %lld, %lld, %lld] must have B, T, h, w >= 1", (long long)B,
                (long long)T, (long long)h, (long long)w);
  if (B * h * w * 64 * 64 > (int64_t)1 << 31 || T > 100000)
    return fail(WANVAE_ESHAPE, "latent shape too large");
  if (int rc = parse_weights(weights, n, m)) return rc;
  return build_topology(m, tp);
}

}  // namespace wanvae

using namespace wanvae;

extern "C" {

const char* wanvae_last_error(void) { return g_err.c_str(); }

int wanvae_profile_enable(int on) {
  g_err.clear();
  g_prof.clear();
  g_prof.on = on != 0;
  return WANVAE_OK;
}

int wanvae_profile_read(int kind, double* ms, int64_t* launches, double* flops, double* bytes) {
  g_err.clear();
  double t = 0, f = 0, by = 0;
  int64_t n = 0;
  for (auto& r : g_prof.recs) {
    if (r.kind != kind) continue;
    HIP_TRY(hipEventSynchronize(r.b));
    float e = 0;
    HIP_TRY(hipEventElapsedTime(&e, r.a, r.b));
    t += e;
    f += r.flops;
    by += r.bytes;
    ++n;
  }
  if (ms) *ms = t;
  if (launches) *launches = n;
  if (flops) *flops = f;
  if (bytes) *bytes = by;
  return WANVAE_OK;
}

int wanvae_set_conv_kernel(int kernel) {
  if (kernel < -1 || kernel >= WANVAE_CONV_KERNELS)
    return fail(WANVAE_EARG, "conv kernel %d is not in -1..%d", kernel, WANVAE_CONV_KERNELS - 1);
  g_conv_kernel.store(kernel);
  return WANVAE_OK;
}

int wanvae_set_norm_kernel(int mode) {
  if (mode < -1 || mode > 1) return fail(WANVAE_EARG, "norm kernel %d is not -1, 0 or 1", mode);
  g_norm_kernel.store(mode);
  return WANVAE_OK;
}

int wanvae_set_decode_pipeline(int on) {
  if (on != 0 && on != 1) return fail(WANVAE_EARG, "decode pipeline switch %d is not 0 or 1", on);
  g_pipeline.store(on);
  return WANVAE_OK;
}

int wanvae_version(void) { return 201; }

int wanvae_decode_workspace_size(int64_t B, int64_t T, int64_t h, int64_t w, const wanvae_tensor* weights,
                                 int64_t n_weights, int32_t dtype, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(WANVAE_EARG, "bytes: NULL");
  WeightMap m;
  Topology tp;
  if (int rc = decode_validate(B, T, h, w, weights, n_weights, dtype, m, tp)) return rc;
  Decoder d(m, tp, dtype, (int)B, (int)T, (int)h, (int)w);
  Arena ar;
  if (int rc = d.plan(ar, nullptr)) return rc;
  *bytes = ar.used;
  return WANVAE_OK;
}

int wanvae_decode(const void* z, int32_t z_dtype, int64_t B, int64_t T, int64_t h, int64_t w,
                  const wanvae_tensor* weights, int64_t n_weights, int32_t dtype, void* video, void* workspace,
                  size_t workspace_bytes, void* stream) {
  g_err.clear();
  WeightMap m;
  Topology tp;
  if (int rc = decode_validate(B, T, h, w, weights, n_weights, dtype, m, tp)) return rc;
  if (int rc = check_dtype(z_dtype, "z_dtype")) return rc;
  if (!z || !video) return fail(WANVAE_EARG, "z and video must not be NULL");
  Decoder measure(m, tp, dtype, (int)B, (int)T, (int)h, (int)w);
  Arena probe;
  measure.plan(probe, nullptr);
  if (workspace && workspace_bytes < probe.used)
    return fail(WANVAE_EWORKSPACE, "workspace of %zu bytes, the decode needs %zu", workspace_bytes, probe.used);
  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (!ws) HIP_TRY(hipMallocAsync(&ws, probe.used, st));
  Decoder d(m, tp, dtype, (int)B, (int)T, (int)h, (int)w);
  Arena ar;
  ar.base = (char*)ws;
  int rc = d.plan(ar, st);
  Pipe* pipe = nullptr;
  if (rc == WANVAE_OK && T > 1 && g_pipeline.load(std::memory_order_relaxed)) rc = pipe_for_device(&pipe);
  if (rc == WANVAE_OK) {
    std::unique_lock<std::mutex> lk;
    if (pipe) lk = std::unique_lock<std::mutex>(pipe->mu);
    rc = d.run(z, z_dtype, video, pipe);
  }
  if (!workspace) {
    hipError_t e = hipFreeAsync(ws, st);
    if (rc == WANVAE_OK && e != hipSuccess) rc = fail(WANVAE_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return rc;
}

// ---------------------------------------------------------------- tiled decode

// The tiled decode of the diffusers PR page on Wan tiling: overlapping spatial tiles of the
// latent, each decoded on its own, composed with a linear ramp over the overlaps.
struct TiledPlan {
  std::vector<std::pair<int, int>> gy, gx;  // (start, size) of the tile rows / columns, latent units
  std::vector<std::vector<int>> groups;     // columns of equal width, decoded as one batch per row
  int F = 0;
  size_t weights = 0, row = 0, stage = 0, acts = 0, total = 0;
};

static std::vector<std::pair<int, int>> tile_axis(int n, int tile_px, int stride_px) {
  std::vector<std::pair<int, int>> g;
  const int t = tile_px / 16, s = stride_px / 16;
  for (int i = 0; i < n; i += s) g.push_back({i, std::min(t, n - i)});
  return g;
}

static int tiled_plan(int64_t B, int64_t T, int64_t h, int64_t w, const wanvae_tensor* weights, int64_t n_weights,
                      int32_t dtype, int32_t tile_h, int32_t tile_w, int32_t stride_h, int32_t stride_w, WeightMap& m,
                      Topology& tp, TiledPlan& P) {
  if (int rc = decode_validate(B, T, h, w, weights, n_weights, dtype, m, tp)) return rc;
  const int32_t sz[4] = {tile_h, tile_w, stride_h, stride_w};
  for (int32_t v : sz)
    if (v < 16 || v % 16 || v > (1 << 20))
      return fail(WANVAE_EARG, "tile %d x %d and stride %d x %d (video pixels) must be positive multiples of 16",
                  tile_h, tile_w, stride_h, stride_w);
  if (stride_h > tile_h || stride_w > tile_w)
    return fail(WANVAE_EARG, "stride %d x %d must not exceed the tile %d x %d", stride_h, stride_w, tile_h, tile_w);
  P.gy = tile_axis((int)h, tile_h, stride_h);
  P.gx = tile_axis((int)w, tile_w, stride_w);
  std::map<int, std::vector<int>> by_w;
  for (int c = 0; c < (int)P.gx.size(); ++c) by_w[-P.gx[c].second].push_back(c);
  for (auto& kv : by_w) P.groups.push_back(kv.second);
  P.F = 4 * (int)T - 3;
  const size_t es = esize(dtype);
  const int thmax = P.gy[0].second;
  {
    Decoder wd(m, tp, dtype, (int)B, (int)T, (int)h, (int)w);
    Arena a;
    if (int rc = wd.plan_weights(a, nullptr)) return rc;
    P.weights = a.used;
  }
  for (auto& g : P.groups) {
    const int tw = P.gx[g[0]].second, nc = (int)g.size();
    P.row += (size_t)B * nc * 3 * P.F * (16 * thmax) * (16 * tw) * es;
    P.stage = std::max(P.stage, (size_t)B * nc * 48 * T * thmax * tw * 4);
    for (size_t r = 0; r < P.gy.size(); ++r) {
      if (r > 0 && P.gy[r].second == P.gy[r - 1].second) continue;
      Decoder d(m, tp, dtype, (int)B * nc, (int)T, P.gy[r].second, tw);
      Arena a;
      if (int rc = d.plan_acts(a)) return rc;
      P.acts = std::max(P.acts, a.used);
    }
  }
  Arena a;
  a.take(P.weights);
  a.take(P.row);
  a.take(P.row);
  a.take(P.stage);
  a.take(P.acts);
  P.total = a.used;
  return WANVAE_OK;
}

int wanvae_decode_tiled_workspace_size(int64_t B, int64_t T, int64_t h, int64_t w, const wanvae_tensor* weights,
                                       int64_t n_weights, int32_t dtype, int32_t tile_h, int32_t tile_w,
                                       int32_t stride_h, int32_t stride_w, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(WANVAE_EARG, "bytes: NULL");
  WeightMap m;
  Topology tp;
  TiledPlan P;
  if (int rc = tiled_plan(B, T, h, w, weights, n_weights, dtype, tile_h, tile_w, stride_h, stride_w, m, tp, P)) return rc;
  *bytes = P.total;
  return WANVAE_OK;
}

int wanvae_decode_tiled(const void* z, int32_t z_dtype, int64_t B, int64_t T, int64_t h, int64_t w,
                        const wanvae_tensor* weights, int64_t n_weights, int32_t dtype, int32_t tile_h, int32_t tile_w,
                        int32_t stride_h, int32_t stride_w, void* video, void* workspace, size_t workspace_bytes,
                        void* stream) {
  g_err.clear();
  WeightMap m;
  Topology tp;
  TiledPlan P;
  if (int rc = tiled_plan(B, T, h, w, weights, n_weights, dtype, tile_h, tile_w, stride_h, stride_w, m, tp, P)) return rc;
  if (int rc = check_dtype(z_dtype, "z_dtype")) return rc;
  if (!z || !video) return fail(WANVAE_EARG, "z and video must not be NULL");
  if (workspace && workspace_bytes < P.total)
    return fail(WANVAE_EWORKSPACE, "workspace of %zu bytes, the tiled decode needs %zu", workspace_bytes, P.total);
  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (!ws) HIP_TRY(hipMallocAsync(&ws, P.total, st));
  int rc = WANVAE_OK;
  {
    Arena ar;
    ar.base = (char*)ws;
    Decoder wd(m, tp, dtype, (int)B, (int)T, (int)h, (int)w);
    rc = wd.plan_weights(ar, st);
    char* rowbuf[2] = {(char*)ar.take(P.row), (char*)ar.take(P.row)};
    char* stage = (char*)ar.take(P.stage);
    char* acts = (char*)ar.take(P.acts);
    Pipe* pipe = nullptr;
    if (rc == WANVAE_OK && T > 1 && g_pipeline.load(std::memory_order_relaxed)) rc = pipe_for_device(&pipe);
    std::unique_lock<std::mutex> lk;
    if (pipe) lk = std::unique_lock<std::mutex>(pipe->mu);
    const size_t es = esize(dtype), zes = esize(z_dtype);
    const int VH = 16 * (int)h, VW = 16 * (int)w;
    const int Ev_max = tile_h - stride_h, Eh_max = tile_w - stride_w;
    std::vector<char*> prev(P.gx.size(), nullptr), cur(P.gx.size(), nullptr);
    int prev_H = 0;
    for (size_t r = 0; r < P.gy.size() && rc == WANVAE_OK; ++r) {
      const int y0 = P.gy[r].first, th = P.gy[r].second, H = 16 * th;
      // decode the row's tiles, one batch per group of equal width (tile k of a group is batch
      // elements k*B .. k*B + B - 1 of that decode)
      size_t off = 0;
      for (const auto& g : P.groups) {
        if (rc != WANVAE_OK) break;
        const int tw = P.gx[g[0]].second, nc = (int)g.size(), W = 16 * tw;
        const size_t zt = (size_t)B * 48 * T * th * tw;  // latent elements of one tile
        const size_t vt = (size_t)B * 3 * P.F * H * W;   // video elements of one tile
        for (int k = 0; k < nc && rc == WANVAE_OK; ++k) {
          hipEvent_t e0 = prof_start(st);
          hipError_t e = launch_crop(z, stage + k * zt * zes, (int)zes, B * 48 * T, (int)h, (int)w, y0,
                                     P.gx[g[k]].first, th, tw, st);
          if (e != hipSuccess) rc = fail(WANVAE_EHIP, "tile crop: %s", hipGetErrorString(e));
          prof_stop(e0, WANVAE_KOTHER, 0, 2.0 * zt * zes, st);
        }
        if (rc != WANVAE_OK) break;
        Decoder d(m, tp, dtype, (int)B * nc, (int)T, th, tw);
        d.use_weights(wd, st);
        Arena aa;
        aa.base = acts;
        char* out = rowbuf[r & 1] + off;
        rc = d.plan_acts(aa);
        if (rc == WANVAE_OK) rc = d.run(stage, z_dtype, out, pipe);
        for (int k = 0; k < nc; ++k) cur[g[k]] = out + k * vt * es;
        off += nc * vt * es;
      }
      // compose the row's tiles in order
      for (size_t c = 0; c < P.gx.size() && rc == WANVAE_OK; ++c) {
        const int x0 = P.gx[c].first, tw = P.gx[c].second, W = 16 * tw;
        TileBlendArgs a;
        a.cur = cur[c];
        a.above = r > 0 ? prev[c] : nullptr;
        a.left = c > 0 ? cur[c - 1] : nullptr;
        a.planes = B * 3 * P.F;
        a.H = H, a.W = W;
        a.Ha = prev_H;
        a.Ev = r > 0 ? std::min({prev_H, H, Ev_max}) : 0;
        a.Wl = c > 0 ? 16 * P.gx[c - 1].second : 0;
        a.Eh = c > 0 ? std::min({a.Wl, W, Eh_max}) : 0;
        a.video = video;
        a.VH = VH, a.VW = VW;
        a.oy = 16 * y0, a.ox = 16 * x0;
        a.keep_h = std::min(stride_h, H), a.keep_w = std::min(stride_w, W);
        hipEvent_t e0 = prof_start(st);
        hipError_t e = launch_tile_blend(a, dtype, st);
        if (e != hipSuccess) rc = fail(WANVAE_EHIP, "tile blend: %s", hipGetErrorString(e));
        prof_stop(e0, WANVAE_KOTHER, 0, 3.0 * a.planes * H * W * es, st);
      }
      std::swap(prev, cur);
      prev_H = H;
    }
  }
  if (!workspace) {
    hipError_t e = hipFreeAsync(ws, st);
    if (rc == WANVAE_OK && e != hipSuccess) rc = fail(WANVAE_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return rc;
}

// ---------------------------------------------------------------- single causal conv

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static int conv_validate(const void* x, const void* cache, int64_t B, int64_t Cin, int64_t t, int64_t h, int64_t w,
                         int64_t n_cache, const wanvae_tensor* weight, const wanvae_tensor* bias, int32_t layout,
                         int32_t dtype, const void* y, int32_t y_dtype, const void* cache_out) {
  if (int rc = check_dtype(dtype, "dtype")) return rc;
  if (int rc = check_dtype(y_dtype, "y_dtype")) return rc;
  if (dtype == kF32 && y_dtype != kF32)
    return fail(WANVAE_EDTYPE, "a float32 conv returns float32 (y_dtype must be WANVAE_F32)");
  if (layout != WANVAE_NCTHW && layout != WANVAE_NTHWC) return fail(WANVAE_EARG, "layout %d unknown", layout);
  if (!x || !y) return fail(WANVAE_EARG, "x and y must not be NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(cache) || !aligned16(cache_out))
    return fail(WANVAE_EARG, "x, cache, y and cache_out must be 16-byte aligned");
  if (y == x || (cache && y == cache) || (cache_out && (cache_out == x || cache_out == y)))
    return fail(WANVAE_EARG, "y must not alias x or cache, and cache_out must not alias x or y");
  if (int rc = check_tensor(weight, "weight")) return rc;
  if (int rc = check_tensor(bias, "bias")) return rc;
  if (B < 1 || Cin < 1 || t < 1 || h < 1 || w < 1) return fail(WANVAE_ESHAPE, "B, Cin, t, h, w must be >= 1");
  if (Cin % 8 != 0) return fail(WANVAE_ESHAPE, "Cin %lld must be a multiple of 8", (long long)Cin);
  if (weight->ndim != 5 || weight->shape[1] != Cin)
    return fail(WANVAE_ESHAPE, "weight %s does not fit Cin %lld", shape_str(weight).c_str(), (long long)Cin);
  const int64_t Cout = weight->shape[0], kt = weight->shape[2], kh = weight->shape[3], kw = weight->shape[4];
  if (Cout < 4 || Cout % 4 != 0) return fail(WANVAE_ESHAPE, "Cout %lld must be a positive multiple of 4", (long long)Cout);
  if ((kt != 1 && kt != 3) || (kh != 1 && kh != 3) || (kw != 1 && kw != 3))
    return fail(WANVAE_ESHAPE, "kernel %lldx%lldx%lld: each extent must be 1 or 3", (long long)kt, (long long)kh,
                (long long)kw);
  if (!shape_is(bias, {Cout})) return fail(WANVAE_ESHAPE, "bias %s, expected [%lld]", shape_str(bias).c_str(), (long long)Cout);
  if (n_cache < 0 || n_cache > 2 || (kt == 1 && n_cache != 0))
    return fail(WANVAE_ESHAPE, "n_cache %lld (needs 0..2, and 0 for kt = 1)", (long long)n_cache);
  if (n_cache > 0 && !cache) return fail(WANVAE_EARG, "cache NULL with n_cache %lld", (long long)n_cache);
  if (cache_out && cache_out == cache && n_cache != 2)
    return fail(WANVAE_EARG, "cache_out may be the cache itself only when both hold 2 frames (n_cache %lld)",
                (long long)n_cache);
  if (t + kt - 1 > kMaxFrames) return fail(WANVAE_ESHAPE, "t %lld too large (at most %d)", (long long)t, kMaxFrames - 2);
  if (B * h * w * (Cin > Cout ? Cin : Cout) > ((int64_t)1 << 31)) return fail(WANVAE_ESHAPE, "frame too large");
  return WANVAE_OK;
}

// frames of the updated cache: the last min(2, n_cache + t) of cache ++ x ("Causal caches")
static int64_t cache_out_frames(int64_t n_cache, int64_t t) { return std::min<int64_t>(2, n_cache + t); }

static size_t conv_ws(int64_t B, int64_t Cin, int64_t Cout, int64_t taps, int64_t t, int64_t h, int64_t w,
                      int64_t n_cache, int32_t layout, int32_t dtype, int32_t y_dtype) {
  Arena ar;
  ar.take((size_t)Cout * taps * Cin * esize(dtype));
  ar.take((size_t)Cout * 4);
  if (layout == WANVAE_NCTHW) {
    ar.take((size_t)(t + n_cache) * B * h * w * Cin * esize(dtype));
    ar.take((size_t)t * B * h * w * Cout * esize(y_dtype));
  }
  take_split(ar, t * B * h * w, Cout);
  return ar.used;
}

// Enqueues the conv on a workspace of at least conv_ws bytes (arguments already validated).
static int conv_run(const void* x, const void* cache, int64_t B, int64_t Cin, int64_t t, int64_t h, int64_t w,
                    int64_t n_cache, const wanvae_tensor* weight, const wanvae_tensor* bias, int32_t layout,
                    int32_t dtype, void* y, int32_t y_dtype, void* cache_out, void* ws, hipStream_t st) {
  const int Cout = (int)weight->shape[0], kt = (int)weight->shape[2], kh = (int)weight->shape[3],
            kw = (int)weight->shape[4];
  Arena ar;
  ar.base = (char*)ws;
  const size_t es = esize(dtype), yes = esize(y_dtype);
  const int64_t hw = h * w;
  const int tpad = 2 * (kt / 2);
  ConvW cw;
  int rc = prep_conv(ar, dtype, weight, bias, Cout, (int)Cin, kt, kh, kw, cw, st);
  FrameRef in, out;
  for (int z = 0; z < tpad - n_cache; ++z) in.push(nullptr, 0);
  void* yout = nullptr;
  if (rc == WANVAE_OK && layout == WANVAE_NCTHW) {
    // convert to frames [n_cache + t][B][h][w][Cin] in the workspace
    void* xin = ar.take((size_t)(t + n_cache) * B * hw * Cin * es);
    yout = ar.take((size_t)t * B * hw * Cout * yes);
    const int64_t fe = B * hw * Cin;
    hipError_t e = hipSuccess;
    if (n_cache)
      e = launch_ncthw_to_frames(cache, dtype, xin, dtype, (int)B, (int)Cin, (int)Cin, (int)n_cache, (int)h, (int)w, st);
    if (e == hipSuccess)
      e = launch_ncthw_to_frames(x, dtype, (char*)xin + n_cache * fe * es, dtype, (int)B, (int)Cin, (int)Cin, (int)t,
                                 (int)h, (int)w, st);
    if (e != hipSuccess) rc = fail(WANVAE_EHIP, "layout conversion: %s", hipGetErrorString(e));
    for (int k = 0; k < n_cache + t; ++k) in.push((char*)xin + k * fe * es, hw * Cin);
    out = frames_of(yout, (int)t, B * hw * Cout, hw * Cout, yes);
  } else if (rc == WANVAE_OK) {
    // [B, frames, h, w, C]: frame k of batch b at base + (b * frames + k) * hwC; read and written in place
    for (int k = 0; k < n_cache; ++k) in.push((char*)cache + k * hw * Cin * es, n_cache * hw * Cin);
    for (int k = 0; k < t; ++k) in.push((char*)x + k * hw * Cin * es, t * hw * Cin);
    out = frames_of(y, (int)t, hw * Cout, t * hw * Cout, yes);
  }
  if (rc == WANVAE_OK) {
    SplitScope scope(take_split(ar, t * B * h * w, Cout));
    ConvCall cc;
    cc.a.mode = y_dtype == dtype ? kEpiFrames : kEpiFramesF32;
    set_out(cc.a, out, Cout);
    rc = run_conv(cw, in, (int)B, (int)h, (int)w, (int)h, (int)w, (int)t, false, cc, dtype, st);
  }
  if (rc == WANVAE_OK && layout == WANVAE_NCTHW) {
    hipError_t e = launch_frames_to_ncthw(yout, y, y_dtype, (int)B, Cout, (int)t, (int)h, (int)w, st);
    if (e != hipSuccess) rc = fail(WANVAE_EHIP, "y layout: %s", hipGetErrorString(e));
  }
  if (rc == WANVAE_OK && cache_out) {
    // the updated cache, frame by frame in order: its frame j is frame n_cache + t - n_out + j
    // of cache ++ x. A row is one (batch, channel) plane (NCTHW) or one batch element (NTHWC).
    // Frame j reads a later or the same frame of the concatenation, so cache_out may be the
    // cache itself (updated in place): each frame's copy is its own launch, in order.
    const int64_t n_out = cache_out_frames(n_cache, t);
    const int64_t fb = (layout == WANVAE_NCTHW ? hw : hw * Cin) * (int64_t)es;  // bytes of a frame in a row
    const int64_t rows = layout == WANVAE_NCTHW ? B * Cin : B;
    for (int64_t j = 0; j < n_out && rc == WANVAE_OK; ++j) {
      const int64_t f = n_cache + t - n_out + j;
      const bool from_cache = f < n_cache;
      const char* src = from_cache ? (const char*)cache + f * fb : (const char*)x + (f - n_cache) * fb;
      const int64_t src_pitch = (from_cache ? n_cache : t) * fb;
      hipEvent_t e0 = prof_start(st);
      hipError_t e = launch_copy_rows(src, src_pitch, (char*)cache_out + j * fb, n_out * fb, fb, rows, st);
      if (e != hipSuccess) rc = fail(WANVAE_EHIP, "cache_out: %s", hipGetErrorString(e));
      prof_stop(e0, WANVAE_KOTHER, 0, 2.0 * fb * rows, st);
    }
  }
  return rc;
}

}  // extern "C"

namespace wanvae {

int conv_plan(const void* x, const void* cache, int64_t B, int64_t Cin, int64_t t, int64_t h, int64_t w,
              int64_t n_cache, const wanvae_tensor* weight, const wanvae_tensor* bias, int32_t layout, int32_t dtype,
              const void* y, int32_t y_dtype, const void* cache_out, size_t* need) {
  g_err.clear();
  if (int rc = conv_validate(x, cache, B, Cin, t, h, w, n_cache, weight, bias, layout, dtype, y, y_dtype, cache_out))
    return rc;
  const int64_t taps = weight->shape[2] * weight->shape[3] * weight->shape[4];
  *need = conv_ws(B, Cin, weight->shape[0], taps, t, h, w, n_cache, layout, dtype, y_dtype);
  return WANVAE_OK;
}

int conv_enqueue(const void* x, const void* cache, int64_t B, int64_t Cin, int64_t t, int64_t h, int64_t w,
                 int64_t n_cache, const wanvae_tensor* weight, const wanvae_tensor* bias, int32_t layout,
                 int32_t dtype, void* y, int32_t y_dtype, void* cache_out, void* ws, hipStream_t st) {
  return conv_run(x, cache, B, Cin, t, h, w, n_cache, weight, bias, layout, dtype, y, y_dtype, cache_out, ws, st);
}

}  // namespace wanvae

extern "C" {

int wanvae_causal_conv3d_workspace_size(int64_t B, int64_t Cin, int64_t Cout, int64_t t, int64_t h, int64_t w,
                                        int64_t n_cache, int32_t layout, int32_t dtype, int32_t y_dtype,
                                        size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(WANVAE_EARG, "bytes: NULL");
  if (int rc = check_dtype(dtype, "dtype")) return rc;
  if (int rc = check_dtype(y_dtype, "y_dtype")) return rc;
  *bytes = conv_ws(B, Cin, Cout, 27, t, h, w, n_cache, layout, dtype, y_dtype);
  return WANVAE_OK;
}

int wanvae_causal_conv3d(const void* x, const void* cache, int64_t B, int64_t Cin, int64_t t, int64_t h, int64_t w,
                         int64_t n_cache, const wanvae_tensor* weight, const wanvae_tensor* bias, int32_t layout,
                         int32_t dtype, void* y, int32_t y_dtype, void* cache_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (int rc = conv_validate(x, cache, B, Cin, t, h, w, n_cache, weight, bias, layout, dtype, y, y_dtype, cache_out))
    return rc;
  const int64_t taps = weight->shape[2] * weight->shape[3] * weight->shape[4];
  const size_t need = conv_ws(B, Cin, weight->shape[0], taps, t, h, w, n_cache, layout, dtype, y_dtype);
  if (workspace && workspace_bytes < need)
    return fail(WANVAE_EWORKSPACE, "workspace of %zu bytes, the conv needs %zu", workspace_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (!ws) HIP_TRY(hipMallocAsync(&ws, need, st));
  int rc = conv_run(x, cache, B, Cin, t, h, w, n_cache, weight, bias, layout, dtype, y, y_dtype, cache_out, ws, st);
  if (!workspace) {
    hipError_t e = hipFreeAsync(ws, st);
    if (rc == WANVAE_OK && e != hipSuccess) rc = fail(WANVAE_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return rc;
}

// ---------------------------------------------------------------- attention block

static int attn_validate(const void* x, int32_t layout, int64_t B, int64_t C, int64_t T, int64_t h, int64_t w,
                         const wanvae_tensor* gamma, const wanvae_tensor* qkv_w, const wanvae_tensor* qkv_b,
                         const wanvae_tensor* proj_w, const wanvae_tensor* proj_b, int32_t dtype, const void* y) {
  if (int rc = check_dtype(dtype, "dtype")) return rc;
  if (layout != WANVAE_NCTHW && layout != WANVAE_NTHWC) return fail(WANVAE_EARG, "layout %d unknown", layout);
  if (!x || !y) return fail(WANVAE_EARG, "x and y must not be NULL");
  if (x == y) return fail(WANVAE_EARG, "y must not alias x");
  const wanvae_tensor* ts[5] = {gamma, qkv_w, qkv_b, proj_w, proj_b};
  const char* nm[5] = {"gamma", "qkv_w", "qkv_b", "proj_w", "proj_b"};
  for (int i = 0; i < 5; ++i)
    if (int rc = check_tensor(ts[i], nm[i])) return rc;
  if (B < 1 || T < 1 || h < 1 || w < 1 || C < 1) return fail(WANVAE_ESHAPE, "B, C, T, h, w must be >= 1");
  if (C % 64 != 0 || C > 1024 || !attn_supported((int)C, dtype))
    return fail(WANVAE_ESHAPE, "C %lld unsupported (64, 128, 256, 384, 512 or 1024)", (long long)C);
  if (numel(gamma) != C) return fail(WANVAE_ESHAPE, "gamma has %lld elements, expected %lld", (long long)numel(gamma), (long long)C);
  if (!(shape_is(qkv_w, {3 * C, C, 1, 1}) || shape_is(qkv_w, {3 * C, C})))
    return fail(WANVAE_ESHAPE, "qkv_w %s, expected [%lld, %lld, 1, 1]", shape_str(qkv_w).c_str(), (long long)(3 * C), (long long)C);
  if (!shape_is(qkv_b, {3 * C})) return fail(WANVAE_ESHAPE, "qkv_b %s", shape_str(qkv_b).c_str());
  if (!(shape_is(proj_w, {C, C, 1, 1}) || shape_is(proj_w, {C, C})))
    return fail(WANVAE_ESHAPE, "proj_w %s, expected [%lld, %lld, 1, 1]", shape_str(proj_w).c_str(), (long long)C, (long long)C);
  if (!shape_is(proj_b, {C})) return fail(WANVAE_ESHAPE, "proj_b %s", shape_str(proj_b).c_str());
  if (B * T * h * w * 3 * C > ((int64_t)1 << 31)) return fail(WANVAE_ESHAPE, "input too large");
  return WANVAE_OK;
}

static size_t attn_ws(int64_t B, int64_t C, int64_t T, int64_t h, int64_t w, int32_t layout, int32_t dtype) {
  Arena ar;
  const size_t es = esize(dtype);
  ar.take((size_t)3 * C * C * es);
  ar.take((size_t)3 * C * 4);
  ar.take((size_t)C * C * es);
  ar.take((size_t)C * 4);
  ar.take((size_t)C * 4);
  AttnBufs ab;
  plan_attn_bufs(ar, ab, (int)(B * T), (int)(h * w), (int)C, dtype, true);
  if (layout == WANVAE_NCTHW) {
    ar.take((size_t)B * T * h * w * C * es);
    ar.take((size_t)B * T * h * w * C * es);
  }
  return ar.used;
}

int wanvae_attn_block_workspace_size(int64_t B, int64_t C, int64_t T, int64_t h, int64_t w, int32_t layout,
                                     int32_t dtype, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(WANVAE_EARG, "bytes: NULL");
  if (int rc = check_dtype(dtype, "dtype")) return rc;
  *bytes = attn_ws(B, C, T, h, w, layout, dtype);
  return WANVAE_OK;
}

int wanvae_attn_block(const void* x, int32_t layout, int64_t B, int64_t C, int64_t T, int64_t h, int64_t w,
                      const wanvae_tensor* gamma, const wanvae_tensor* qkv_w, const wanvae_tensor* qkv_b,
                      const wanvae_tensor* proj_w, const wanvae_tensor* proj_b, int32_t dtype, void* y,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (int rc = attn_validate(x, layout, B, C, T, h, w, gamma, qkv_w, qkv_b, proj_w, proj_b, dtype, y)) return rc;
  const size_t need = attn_ws(B, C, T, h, w, layout, dtype);
  if (workspace && workspace_bytes < need)
    return fail(WANVAE_EWORKSPACE, "workspace of %zu bytes, the block needs %zu", workspace_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (!ws) HIP_TRY(hipMallocAsync(&ws, need, st));
  Arena ar;
  ar.base = (char*)ws;
  const size_t es = esize(dtype);
  const int Ci = (int)C, nfr = (int)(B * T), S = (int)(h * w);
  int rc = WANVAE_OK;
  ConvW qkv, proj;
  float* g = nullptr;
  rc = prep_conv(ar, dtype, qkv_w, qkv_b, 3 * Ci, Ci, 1, 1, 1, qkv, st);
  if (rc == WANVAE_OK) rc = prep_conv(ar, dtype, proj_w, proj_b, Ci, Ci, 1, 1, 1, proj, st);
  if (rc == WANVAE_OK) rc = prep_vec(ar, dtype, gamma, Ci, g, st);
  AttnBufs ab;
  plan_attn_bufs(ar, ab, nfr, S, Ci, dtype, true);
  SplitScope scope(ab.split);
  // frames folded into the batch: frame index b' = t * B + b (NCTHW, converted) or b * T + t (NTHWC)
  const void* xf = x;
  void* yf = y;
  if (rc == WANVAE_OK && layout == WANVAE_NCTHW) {
    void* xb = ar.take((size_t)nfr * S * Ci * es);
    yf = ar.take((size_t)nfr * S * Ci * es);
    hipError_t e = launch_ncthw_to_frames(x, dtype, xb, dtype, (int)B, Ci, Ci, (int)T, (int)h, (int)w, st);
    if (e != hipSuccess) rc = fail(WANVAE_EHIP, "x layout: %s", hipGetErrorString(e));
    xf = xb;
  }
  if (rc == WANVAE_OK) {
    const FrameRef xr = frames_of(const_cast<void*>(xf), 1, 0, (int64_t)S * Ci, es);
    const FrameRef yr = frames_of(yf, 1, 0, (int64_t)S * Ci, es);
    rc = run_attn(xr, yr, nfr, (int)h, (int)w, Ci, g, qkv, proj, ab, dtype, st);
  }
  if (rc == WANVAE_OK && layout == WANVAE_NCTHW) {
    hipError_t e = launch_frames_to_ncthw(yf, y, dtype, (int)B, Ci, (int)T, (int)h, (int)w, st);
    if (e != hipSuccess) rc = fail(WANVAE_EHIP, "y layout: %s", hipGetErrorString(e));
  }
  if (!workspace) {
    hipError_t e = hipFreeAsync(ws, st);
    if (rc == WANVAE_OK && e != hipSuccess) rc = fail(WANVAE_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return rc;
}

}  // extern "C"
