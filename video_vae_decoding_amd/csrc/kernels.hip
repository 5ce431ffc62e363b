// gfx950 kernels of the Wan2.2 TI2V-5B VAE decoder.
//
//  k_conv_halo  bf16 3x3 causal convs (3x3x3 and the upsampling 3x3): a workgroup copies the
//               input patch under its block of positions into LDS once per (time tap,
//               channel block) and the nine spatial taps read shifted windows of it; the taps
//               run column shift by column shift, so a wave reads each patch row once per
//               shift and keeps it in registers for the three tap rows that use it.
//  k_conv_dma   implicit-GEMM conv with tiles copied straight to LDS: in bf16 the other
//               shapes (1x1 shortcuts, 3x1x1 time convs, conv_in, the attention's 1x1 convs),
//               in fp32 every conv with more than 64 output channels.
//  k_conv       the same GEMM with register-staged loads, for small Cout.
//               All conv kernels accumulate in fp32 (v_mfma_f32_16x16x32_bf16 in bf16,
//               v_mfma_f32_16x16x4f32 in fp32) and fuse the epilogues: bias, residual add,
//               DupUp3D add, the time conv's channel->frame interleave, unpatchify + clamp,
//               and the q/k/v split.
//  k_norm_v     WanRMS_norm (+ SiLU) per position; the bf16 chain is evaluated to about a
//               float32 ulp before each bf16 rounding. On large launches the bf16 SiLU comes
//               from a table of its results in LDS, which leaves the pass streaming at about
//               the device-copy rate.
//  k_attn_mm    bf16 single-head attention over the h*w positions of a frame on materialised
//  k_attn_fac   scores: the scores GEMM with each 128-key tile's softmax in its epilogue (P
//               stored in bf16), the per-tile weights, and the P V GEMM with a running rescale.
//  k_attn       the fp32 attention, flash style: the head dim is split across the waves of a
//               workgroup, partial scores are summed through LDS in a fixed order, online
//               softmax (per wave over the whole tile, or per wave over its own query rows
//               with P shared through LDS).
// The tiled decode's crop and blend kernels are in tiles.hip.
// Reference for what is computed: FastVideo's "wan22_vae_decode reference.py" page
// (sections "The parts" and "Precision").
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "internal.h"

namespace wanvae {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

struct bf16_t {
  uint16_t u;
};

// ------------------------------------------------------------------ element helpers

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

// float -> bfloat16, round to nearest even, NaN stays NaN (gfx950's v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two floats -> two bfloat16 in one 32-bit word (low half = a), one conversion instruction
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ float R(float v) { return v; }
  static __device__ __forceinline__ void ld4(const float* p, float v[4]) {
    float4 x = *(const float4*)p;
    v[0] = x.x, v[1] = x.y, v[2] = x.z, v[3] = x.w;
  }
  static __device__ __forceinline__ void st4(float* p, const float v[4]) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
};
template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(p->u); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { p->u = f2bf(v); }
  static __device__ __forceinline__ float R(float v) { return bf2f(f2bf(v)); }
  static __device__ __forceinline__ void ld4(const bf16_t* p, float v[4]) {
    uint2 x = *(const uint2*)p;
    v[0] = bf2f(x.x & 0xffff), v[1] = bf2f(x.x >> 16), v[2] = bf2f(x.y & 0xffff), v[3] = bf2f(x.y >> 16);
  }
  static __device__ __forceinline__ void st4(bf16_t* p, const float v[4]) {
    uint2 x;
    x.x = pack2_bf16(v[0], v[1]);
    x.y = pack2_bf16(v[2], v[3]);
    *(uint2*)p = x;
  }
};

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). Renumber
// them so that each XCD runs a contiguous range of tiles, which share input rows and
// weight tiles in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int X = 8;
  const int q = n / X, r = n % X, xcd = bid % X, idx = bid / X;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// One 16x16 MFMA step on a 16-byte fragment pair: bf16 covers 32 k (8 per lane group),
// fp32 covers 16 k (4 per lane group, one MFMA per component). The k order inside a
// fragment is the same for both operands, so the sum is the same contraction.
template <typename T>
struct Mma;
template <>
struct Mma<bf16_t> {
  static __device__ __forceinline__ void run(f32x4_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  acc, 0, 0, 0);
  }
};
template <>
struct Mma<float> {
  static __device__ __forceinline__ void run(f32x4_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// ------------------------------------------------------------------ conv epilogue

// v[0..3]: accumulated sums + bias for output channels c..c+3 at (frame t, batch b, y, x).
// Slot of key pix in a frame's row of V^T: within each block of 32 keys, key 16 kt + 4 g + e
// (kt < 2, g < 4, e < 4) sits at 8 g + 4 kt + e. One lane of the attention's P V product
// takes keys 4g..4g+3 of both 16-key halves of a block, which are then one 16-byte vector.
__device__ __forceinline__ int vt_slot(int pix) {
  const int r = pix & 31;
  return (pix & ~31) | ((r & 12) << 1) | ((r & 16) >> 2) | (r & 3);
}

template <typename T>
__device__ __forceinline__ void conv_epilogue(const ConvArgs& a, int t, int b, int y, int x, int c, float v[4]) {
  using X = Elem<T>;
  if (a.mode == kEpiFramesF32) {
    // the float32 sums + bias, unrounded, as float32 frames (c and outC are multiples of 4)
    float* o = (float*)a.out[t] + b * a.out_bs[t] + ((int64_t)y * a.Wo + x) * a.outC + c;
    *(float4*)o = make_float4(v[0], v[1], v[2], v[3]);
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = X::R(v[i]);
  const int64_t pix = (int64_t)y * a.Wo + x;
  if (a.has_res) {
    const T* r = (const T*)a.res[t] + b * a.res_bs[t] + pix * a.outC + c;
    float rv[4];
    X::ld4(r, rv);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = X::R(v[i] + rv[i]);
  }
  if (a.has_dup) {
    // DupUp3D: dup[c, ft*t + s, 2y + i, 2x + j] = in[(4 ft c + 4 s + 2 i + j) / r, t, y, x]
    const int ts = t + a.dup_shift, tin = ts / a.dup_ft, sub_t = ts - tin * a.dup_ft;
    const int Wh = a.Wo >> 1;
    const T* d = (const T*)a.dup[tin] + b * a.dup_bs[tin] + ((int64_t)(y >> 1) * Wh + (x >> 1)) * a.dup_C;
    const int sub = 4 * sub_t + 2 * (y & 1) + (x & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = X::R(v[i] + X::ld(d + (4 * a.dup_ft * (c + i) + sub) / a.dup_r));
  }
  if (a.mode == kEpiFrames) {
    X::st4((T*)a.out[t] + b * a.out_bs[t] + pix * a.outC + c, v);
  } else if (a.mode == kEpiInterleave) {
    const int half = c >= a.outC ? 1 : 0, fr = 2 * t + half;
    X::st4((T*)a.out[fr] + b * a.out_bs[fr] + pix * a.outC + (c - half * a.outC), v);
  } else if (a.mode == kEpiVideo) {
    // video[b, k, f, 2y + i, 2x + j] = clamp(out[b, 4k + 2j + i, f, y, x]); NaN passes through
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int cc = c + e;
      if (cc >= a.Cout) break;
      const int k = cc >> 2, j = (cc >> 1) & 1, i = cc & 1;
      const float u = v[e] < -1.f ? -1.f : (v[e] > 1.f ? 1.f : v[e]);
      T* o = (T*)a.video + ((((int64_t)b * 3 + k) * a.vF + a.vf0 + t) * (2 * a.Ho) + 2 * y + i) * (int64_t)(2 * a.Wo) +
             2 * x + j;
      X::st(o, u);
    }
  } else {  // kEpiQKV
    const int C = a.outC, fr = t * a.B + b;
    if (c < 2 * C) {
      T* o = (T*)(c < C ? a.q : a.k) + ((int64_t)fr * a.S + pix) * C + (c < C ? c : c - C);
      X::st4(o, v);
    } else {
      T* o = (T*)a.vt + ((int64_t)fr * C + (c - 2 * C)) * a.Sp + vt_slot(pix);
#pragma unroll
      for (int e = 0; e < 4; ++e) X::st(o + (int64_t)e * a.Sp, v[e]);
    }
  }
}

// 256 bytes of zeros in device memory: the source of every load that stands for padding,
// a missing history frame or a channel beyond the tensor (never written).
// 4 KB: a load that stands for a zero row may also add the row's channel-block offset
// (at most 2 KB for 1024 channels) to it and still read zeros.
static __device__ __attribute__((aligned(256))) uint4 g_zero_page[256];

// ------------------------------------------------------------------ implicit-GEMM conv
//
// GEMM view: D[n][m] = sum_k W[n][k] * A[m][k], n = output channel, m = output position
// (t, b, y, x), k = (tap, input channel). Each workgroup (4 waves, 2 x 2) computes a TC x TP
// tile of D. Per K step (one tap, BK input channels = 128 bytes per row) the W and A tiles
// are staged through LDS (double buffered, one barrier per step): each thread loads 16-byte
// chunks from HBM/L2 for step s+1 into registers while the MFMAs of step s run. A rows are
// gathered from the frame table with the tap's shift (zero outside the frame or for a
// missing history frame), so neither padding nor the cache concatenation is materialised.
// Weights are the MFMA A operand: every lane then holds 4 consecutive output channels.
template <typename T, int TC, int TP>
__global__ void __launch_bounds__(256) k_conv(const ConvArgs a) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int BK = 8 * VEC;
  constexpr int ROW = 144;  // 128 data bytes + 16 pad: conflict-free 16-byte LDS reads
  constexpr int NWR = TC / 32, NAR = TP / 32;
  constexpr int STAGE = (TC + TP) * ROW;
  constexpr int WC = TC / 2, WP = TP / 2, TCN = WC / 16, TPN = WP / 16;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int HWo = a.Ho * a.Wo;
  const int M = a.F * a.B * HWo;
  const int nct = (a.Cout + TC - 1) / TC;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int ct = bid % nct, pt = bid / nct;
  const int c0 = ct * TC, m0 = pt * TP;
  const int j = tid & 7, r0 = tid >> 3;
  const int khw = a.kh * a.kw, taps = a.kt * khw;
  const int csteps = (a.Cin + BK - 1) / BK;
  const int steps = taps * csteps;
  const int64_t Ktot = (int64_t)taps * a.Cin;
  const int ph = a.kh >> 1, pw = a.kw >> 1;

  // per A row: the row's frame pointer for each time tap, and its output (y, x)
  const T* rb0[NAR];
  const T* rb1[NAR];
  const T* rb2[NAR];
  int ry[NAR], rx[NAR];
#pragma unroll
  for (int i = 0; i < NAR; ++i) {
    const int m = m0 + r0 + 32 * i;
    rb0[i] = rb1[i] = rb2[i] = nullptr;
    ry[i] = rx[i] = 0;
    if (m < M) {
      const int x = m % a.Wo;
      int q = m / a.Wo;
      const int y = q % a.Ho;
      q /= a.Ho;
      const int b = q % a.B, t = q / a.B;
      ry[i] = y;
      rx[i] = x;
      const T* p0 = (const T*)a.in[t];
      rb0[i] = p0 ? p0 + b * a.in_bs[t] : nullptr;
      if (a.kt > 1) {
        const T* p1 = (const T*)a.in[t + 1];
        const T* p2 = (const T*)a.in[t + 2];
        rb1[i] = p1 ? p1 + b * a.in_bs[t + 1] : nullptr;
        rb2[i] = p2 ? p2 + b * a.in_bs[t + 2] : nullptr;
      }
    }
  }

  // K steps in order: taps (dt, dy, dx) major, blocks of BK input channels minor. The cursor
  // (the next step to load) advances without divisions; per tap it recomputes each A row's
  // pointer to the tap's input pixel (nullptr where the tap reads zeros).
  const T* wrow[NWR];
#pragma unroll
  for (int i = 0; i < NWR; ++i) {
    const int n = c0 + r0 + 32 * i;
    wrow[i] = n < a.Cout ? (const T*)a.w + n * Ktot + j * VEC : nullptr;
  }
  const T* ap[NAR];
  int cdt = 0, cdy = 0, cdx = 0, ccs = 0;
  int64_t woff = 0;
  auto set_tap = [&]() {
#pragma unroll
    for (int i = 0; i < NAR; ++i) {
      const T* base = cdt == 0 ? rb0[i] : (cdt == 1 ? rb1[i] : rb2[i]);
      int yy, xx;
      bool ok = base != nullptr;
      if (a.up) {
        const int yu = ry[i] + cdy - ph, xu = rx[i] + cdx - pw;
        ok = ok && yu >= 0 && yu < a.Ho && xu >= 0 && xu < a.Wo;
        yy = yu >> 1;
        xx = xu >> 1;
      } else {
        yy = ry[i] + cdy - ph;
        xx = rx[i] + cdx - pw;
        ok = ok && yy >= 0 && yy < a.Hin && xx >= 0 && xx < a.Win;
      }
      ap[i] = ok ? base + ((int64_t)yy * a.Win + xx) * a.Cin + j * VEC : nullptr;
    }
  };
  auto advance = [&]() {
    if (++ccs == csteps) {
      ccs = 0;
      woff += a.Cin;
      if (++cdx == a.kw) {
        cdx = 0;
        if (++cdy == a.kh) {
          cdy = 0;
          ++cdt;
        }
      }
      set_tap();
    }
  };
  uint4 wr[NWR], ar[NAR];
  // unconditional 16-byte loads: a lane whose chunk is zero reads the zero page instead
  const uint4* zero = g_zero_page;
  auto gload = [&]() {
    const int cb = ccs * BK;
    const bool cok = cb + j * VEC < a.Cin;
#pragma unroll
    for (int i = 0; i < NWR; ++i) wr[i] = *((cok && wrow[i]) ? (const uint4*)(wrow[i] + woff + cb) : zero);
#pragma unroll
    for (int i = 0; i < NAR; ++i) ar[i] = *((cok && ap[i]) ? (const uint4*)(ap[i] + cb) : zero);
  };
  auto sstore = [&](int buf) {
    char* sw = smem + buf * STAGE;
    char* sa = sw + TC * ROW;
#pragma unroll
    for (int i = 0; i < NWR; ++i) *(uint4*)(sw + (r0 + 32 * i) * ROW + j * 16) = wr[i];
#pragma unroll
    for (int i = 0; i < NAR; ++i) *(uint4*)(sa + (r0 + 32 * i) * ROW + j * 16) = ar[i];
  };

  const int wc = wave >> 1, wp = wave & 1;
  f32x4_t acc[TCN][TPN];
#pragma unroll
  for (int ic = 0; ic < TCN; ++ic)
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) acc[ic][ip] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A step is two halves of 64 bytes per row. Fragments come in two register sets: the second
  // half's are read while the first half's MFMAs run, and the next step's first half (after
  // the barrier that publishes it) while the second half's run.
  uint4 wf[2][TCN], af[2][TPN];
  auto read_half = [&](int set, int buf, int sub) {
    const char* sw = smem + buf * STAGE + (wc * WC) * ROW;
    const char* sa = smem + buf * STAGE + TC * ROW + (wp * WP) * ROW;
    const int off = (sub * 4 + (lane >> 4)) * 16;
#pragma unroll
    for (int ic = 0; ic < TCN; ++ic) wf[set][ic] = *(const uint4*)(sw + (ic * 16 + (lane & 15)) * ROW + off);
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) af[set][ip] = *(const uint4*)(sa + (ip * 16 + (lane & 15)) * ROW + off);
  };
  auto mfma_half = [&](int set) {
#pragma unroll
    for (int ic = 0; ic < TCN; ++ic)
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip) Mma<T>::run(acc[ic][ip], wf[set][ic], af[set][ip]);
  };

  set_tap();
  gload();
  sstore(0);
  __syncthreads();
  read_half(0, 0, 0);
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    if (s + 1 < steps) {
      advance();
      gload();
    }
    read_half(1, buf, 1);
    mfma_half(0);
    if (s + 1 < steps) sstore(buf ^ 1);
    __syncthreads();
    if (s + 1 < steps) read_half(0, buf ^ 1, 0);
    mfma_half(1);
  }

#pragma unroll
  for (int ip = 0; ip < TPN; ++ip) {
    const int m = m0 + wp * WP + ip * 16 + (lane & 15);
    if (m >= M) continue;
    const int x = m % a.Wo;
    int q = m / a.Wo;
    const int y = q % a.Ho;
    q /= a.Ho;
    const int b = q % a.B, t = q / a.B;
#pragma unroll
    for (int ic = 0; ic < TCN; ++ic) {
      const int c = c0 + wc * WC + ic * 16 + 4 * (lane >> 4);
      if (c >= a.Cout) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[ic][ip][e] + (c + e < a.Cout ? a.bias[c + e] : 0.f);
      conv_epilogue<T>(a, t, b, y, x, c, v);
    }
  }
}

// 8 consecutive output channels c..c+7 (already bias-added and rounded to bf16) at (t, b, y, x):
// residual and DupUp3D sums (each rounded) and the store, for the frame / interleave / q-k-vT
// epilogues. Requires Cout and outC multiples of 8.
__device__ __forceinline__ uint4 pack8_bf16(const float v[8]) {
  uint4 r;
  r.x = pack2_bf16(v[0], v[1]);
  r.y = pack2_bf16(v[2], v[3]);
  r.z = pack2_bf16(v[4], v[5]);
  r.w = pack2_bf16(v[6], v[7]);
  return r;
}

__device__ __forceinline__ void unpack8_bf16(const uint4 r, float v[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf2f(w[e] & 0xffff);
    v[2 * e + 1] = bf2f(w[e] >> 16);
  }
}

// A 16-byte store marked non-temporal (streamed past the caches' keep policy): a conv's
// output is not read again before it leaves L2.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16_nt(void* p, const uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, (u32x4_t*)p);
}

__device__ __forceinline__ void epilogue8_bf16(const ConvArgs& a, int t, int b, int y, int x, int c, float v[8]) {
  using T = bf16_t;
  const int64_t pix = (int64_t)y * a.Wo + x;
  if (a.has_res) {
    float r[8];
    unpack8_bf16(*(const uint4*)((const T*)a.res[t] + b * a.res_bs[t] + pix * a.outC + c), r);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf2f(f2bf(v[e] + r[e]));
  }
  if (a.has_dup) {
    const int ts = t + a.dup_shift, tin = ts / a.dup_ft, sub_t = ts - tin * a.dup_ft;
    const T* d = (const T*)a.dup[tin] + b * a.dup_bs[tin] + ((int64_t)(y >> 1) * (a.Wo >> 1) + (x >> 1)) * a.dup_C;
    const int sub = 4 * sub_t + 2 * (y & 1) + (x & 1);
    float dv[8];
    if (a.dup_r == 4 * a.dup_ft) {
      // each input channel repeated over exactly the (ft, 2, 2) sub-positions: channel c
      unpack8_bf16(*(const uint4*)(d + c), dv);
    } else if (2 * a.dup_r == 4 * a.dup_ft) {
      // twice the input channels of the output (up block 2): output channel c + e takes input
      // channel 2 (c + e) + sub / r, every other one of the 16 from 2c on (32 bytes, aligned)
      const uint4 q0 = *(const uint4*)(d + 2 * c), q1 = *(const uint4*)(d + 2 * c + 8);
      const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const bool odd = sub >= a.dup_r;
#pragma unroll
      for (int e = 0; e < 8; ++e) dv[e] = __uint_as_float(odd ? w[e] & 0xffff0000u : w[e] << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dv[e] = bf2f(d[(4 * a.dup_ft * (c + e) + sub) / a.dup_r].u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf2f(f2bf(v[e] + dv[e]));
  }
  if (a.mode == kEpiFrames) {
    st16_nt((T*)a.out[t] + b * a.out_bs[t] + pix * a.outC + c, pack8_bf16(v));
  } else if (a.mode == kEpiInterleave) {
    const int half = c >= a.outC ? 1 : 0, fr = 2 * t + half;
    st16_nt((T*)a.out[fr] + b * a.out_bs[fr] + pix * a.outC + (c - half * a.outC), pack8_bf16(v));
  } else if (a.mode == kEpiQKV) {
    const int C = a.outC, fr = t * a.B + b;
    if (c < 2 * C) {
      *(uint4*)((T*)(c < C ? a.q : a.k) + ((int64_t)fr * a.S + pix) * C + (c < C ? c : c - C)) = pack8_bf16(v);
    } else {
      T* o = (T*)a.vt + ((int64_t)fr * C + (c - 2 * C)) * a.Sp + vt_slot(pix);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[(int64_t)e * a.Sp].u = f2bf(v[e]);
    }
  }
}

// ------------------------------------------------------------------ implicit-GEMM conv, LDS-DMA pipeline (bf16)
//
// The same GEMM as k_conv, for bf16 operands, with the global -> LDS copies done by the
// gfx950 direct-to-LDS loads (global_load_lds_dwordx4: each lane moves 16 bytes from its own
// global address into LDS at base + 16 * lane, with no register round trip). K steps are 32
// input channels of one tap (64-byte rows of 4 chunks). STAGES LDS buffers form a pipeline:
// the loads for step s + STAGES - 1 are in flight while the MFMAs of step s run; each wave
// waits only for its own loads of step s (s_waitcnt vmcnt) before the workgroup barrier.
// Rows are stored with their 4 chunks permuted, slot = chunk ^ ((row >> 1) & 3), so that the
// 16-byte LDS reads of an MFMA fragment (16 rows, one chunk) hit distinct banks. Taps that
// fall in the padding, on a missing history frame, or beyond Cin/Cout load from a zero page.

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate (gfx9 encoding): vmcnt <= n, lgkmcnt <= 0, expcnt unconstrained
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

template <int TC, int TP, int WGC, int WGP, int STAGES, int MINB, bool ALIGNED, bool RB2 = false, typename T = bf16_t>
__global__ void __launch_bounds__(64 * WGC * WGP, MINB) k_conv_dma(const ConvArgs a) {
  // ALIGNED: Cin % KS == 0, Cout % TC == 0 and TC >= 16 * waves, so every weight row a wave
  // loads exists and no 16-byte chunk straddles the end of a pixel: the per-step loads need
  // no selects. T is bf16_t (32 channels per K step) or float (16).
  constexpr int NWAVE = WGC * WGP;
  constexpr int ROWB = 64;                       // bytes per row per step
  constexpr int ES = (int)sizeof(T), KS = ROWB / ES, CE = 16 / ES;  // element size, channels per step, per chunk
  constexpr int WC = TC / WGC, WP = TP / WGP;    // wave tile
  constexpr int TCN = WC / 16, TPN = WP / 16;
  // DMA instructions per wave per step (each moves 16 rows): W, A. When the W tile has fewer
  // than 16 * NWAVE rows, the waves past it load the zero page into a spare LDS slot, so that
  // every wave has the same number of loads in flight (the vmcnt waits count them).
  constexpr int NIW = TC >= 16 * NWAVE ? TC / (16 * NWAVE) : 1;
  constexpr int NIA = TP / (16 * NWAVE);
  constexpr int NI = NIW + NIA;
  constexpr int SPARE = TC >= 16 * NWAVE ? 0 : 1024;
  constexpr int SW = TC * ROWB, SA = TP * ROWB, STAGE = SW + SA + SPARE;
  static_assert((TC < 16 * NWAVE || NIW * 16 * NWAVE == TC) && NIA * 16 * NWAVE == TP, "tile / wave mismatch");
  static_assert(TC % 16 == 0, "W tile rows");
  static_assert(!ALIGNED || TC >= 16 * NWAVE, "the aligned path has no spare weight rows");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  __shared__ __attribute__((aligned(1024))) char s0[STAGE];
  __shared__ __attribute__((aligned(1024))) char s1[STAGE];
  __shared__ __attribute__((aligned(1024))) char s2[STAGES > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char s3[STAGES > 3 ? STAGE : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets are scalar
  const int HWo = a.Ho * a.Wo;
  const int M = a.F * a.B * HWo;
  const int nct = (a.Cout + TC - 1) / TC;
  const int ntiles = nct * ((M + TP - 1) / TP);
  // split K: workgroup z of a.ksplit takes the z-th contiguous range of K steps; the tiles of
  // one range are adjacent (they share its weight rows)
  const int bid0 = xcd_remap(blockIdx.x, gridDim.x);
  const int kz = __builtin_amdgcn_readfirstlane(bid0 / ntiles), bid = bid0 - kz * ntiles;
  const int ct = bid % nct, pt = bid / nct;
  const int c0 = ct * TC, m0 = pt * TP;
  const int khw = a.kh * a.kw, taps = a.kt * khw;
  const int csteps = (a.Cin + KS - 1) / KS;
  const int all_steps = taps * csteps;
  const int s_begin = (int)((int64_t)all_steps * kz / a.ksplit);
  const int steps = (int)((int64_t)all_steps * (kz + 1) / a.ksplit) - s_begin;
  const int64_t Ktot = (int64_t)taps * a.Cin;
  const int ph = a.kh >> 1, pw = a.kw >> 1;
  const char* zero = (const char*)g_zero_page;

  // this lane's DMA slots: row r = base + lane / 4, slot lane % 4 holding chunk slot ^ swz
  const int lrow = lane >> 2, lslot = lane & 3;
  const int lchunk = lslot ^ ((lrow >> 1) & 3);
  // W rows: instruction i covers tile rows (wave * NIW + i) * 16 .. + 15. Aligned: the byte
  // offset of this lane's chunk from the tile's first weight row is fixed; a scalar base
  // advances by the step's K offset.
  const char* wtile = (const char*)((const T*)a.w + (int64_t)c0 * Ktot);
  uint32_t woffl[NIW];
  const T* wrow[NIW];
  int wdst[NIW];  // LDS offset of the instruction's 16 rows (the spare slot past the W tile)
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int r = (wave * NIW + i) * 16;
    const int n = c0 + r + lrow;
    woffl[i] = (uint32_t)(((int64_t)(r + lrow) * Ktot + lchunk * CE) * ES);
    wrow[i] = (r < TC && n < a.Cout) ? (const T*)a.w + n * Ktot + lchunk * CE : nullptr;
    wdst[i] = r < TC ? r * ROWB : SW + SA;
  }
  // A rows: position, and its frame for each time tap
  const T* rb0[NIA];
  const T* rb1[NIA];
  const T* rb2[NIA];
  int ry[NIA], rx[NIA];
#pragma unroll
  for (int i = 0; i < NIA; ++i) {
    const int m = m0 + (wave * NIA + i) * 16 + lrow;
    rb0[i] = rb1[i] = rb2[i] = nullptr;
    ry[i] = rx[i] = 0;
    if (m < M) {
      const int x = m % a.Wo;
      int q = m / a.Wo;
      const int y = q % a.Ho;
      q /= a.Ho;
      const int b = q % a.B, t = q / a.B;
      ry[i] = y;
      rx[i] = x;
      const T* p0 = (const T*)a.in[t];
      rb0[i] = p0 ? p0 + b * a.in_bs[t] : nullptr;
      if (a.kt > 1) {
        const T* p1 = (const T*)a.in[t + 1];
        const T* p2 = (const T*)a.in[t + 2];
        rb1[i] = p1 ? p1 + b * a.in_bs[t + 1] : nullptr;
        rb2[i] = p2 ? p2 + b * a.in_bs[t + 2] : nullptr;
      }
    }
  }

  // issue cursor: the next K step to load (taps major, KS-channel blocks minor), advanced
  // without divisions; per tap each A row's source pointer (the zero page where the tap reads
  // zeros: padding, a missing history frame, a position past the end)
  const char* ap[NIA];
  // the cursor starts at step s_begin: tap s_begin / csteps, channel block s_begin % csteps
  const int tap0 = s_begin / csteps;
  int ccs = s_begin - tap0 * csteps;
  int cdt = tap0 / khw;
  int cdy = (tap0 - cdt * khw) / a.kw;
  int cdx = tap0 - cdt * khw - cdy * a.kw;
  int64_t woff = (int64_t)tap0 * a.Cin;
  auto set_tap = [&]() {
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
      const T* base = cdt == 0 ? rb0[i] : (cdt == 1 ? rb1[i] : rb2[i]);
      int yy, xx;
      bool ok = base != nullptr;
      if (a.up) {
        const int yu = ry[i] + cdy - ph, xu = rx[i] + cdx - pw;
        ok = ok && yu >= 0 && yu < a.Ho && xu >= 0 && xu < a.Wo;
        yy = yu >> 1;
        xx = xu >> 1;
      } else {
        yy = ry[i] + cdy - ph;
        xx = rx[i] + cdx - pw;
        ok = ok && yy >= 0 && yy < a.Hin && xx >= 0 && xx < a.Win;
      }
      ap[i] = ok ? (const char*)(base + ((int64_t)yy * a.Win + xx) * a.Cin + lchunk * CE) : zero + lchunk * 16;
    }
  };
  auto advance = [&]() {
    if (++ccs == csteps) {
      ccs = 0;
      woff += a.Cin;
      if (++cdx == a.kw) {
        cdx = 0;
        if (++cdy == a.kh) {
          cdy = 0;
          ++cdt;
        }
      }
      set_tap();
    }
  };
  auto issue = [&](char* buf) {
    const int cb = ccs * KS;
    if constexpr (ALIGNED) {
      const char* wstep = wtile + (woff + cb) * ES;
#pragma unroll
      for (int i = 0; i < NIW; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(wstep + woffl[i]), LDS_PTR(buf + wdst[i]), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < NIA; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(ap[i] + cb * ES), LDS_PTR(buf + SW + (wave * NIA + i) * 1024), 16,
                                         0, 0);
    } else {
      const bool cok = cb + lchunk * CE < a.Cin;
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const char* src = (cok && wrow[i]) ? (const char*)(wrow[i] + woff + cb) : zero;
        __builtin_amdgcn_global_load_lds((const void*)src, LDS_PTR(buf + wdst[i]), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NIA; ++i) {
        const char* src = cok ? ap[i] + cb * ES : zero;
        __builtin_amdgcn_global_load_lds((const void*)src, LDS_PTR(buf + SW + (wave * NIA + i) * 1024), 16, 0, 0);
      }
    }
    advance();
  };

  const int wc = wave / WGP, wp = wave % WGP;
  f32x4_t acc[TCN][TPN];
#pragma unroll
  for (int ic = 0; ic < TCN; ++ic)
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) acc[ic][ip] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // fragment reads: row base + (lane & 15), logical chunk lane >> 4
  const int rslot = ((lane >> 4) ^ (((lane & 15) >> 1) & 3)) * 16 + (lane & 15) * ROWB;
  // waits until this wave's loads of step s are done (at most the later steps' pending) and
  // its LDS reads have returned, then the workgroup barrier: step s's tile is complete in LDS
  // for every wave, and every wave is done reading the buffers of the steps before s - 1
  auto sync_step = [&](int s) {
    if (s + STAGES - 2 < steps)
      wait_vm_lgkm0<NI * (STAGES - 2)>();
    else
      wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
  };
  char* bufs[4] = {s0, s1, s2, s3};
  if constexpr (RB2) {
    // One wave per SIMD: two register sets of fragments. The MFMAs of step s (set s & 1)
    // are interleaved with the LDS reads of step s + 1 into the other set, so the read
    // latency hides behind the matrix pipe without a second wave. The barrier of step s + 1
    // comes first: after it, no wave reads the buffer of step s any more (its fragments are
    // in registers), and the DMA of step s + STAGES refills it.
    uint4 wf[2][TCN], af[2][TPN];
    auto rd = [&](int set, const char* buf) {
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) wf[set][ic] = *(const uint4*)(buf + (wc * WC + ic * 16) * ROWB + rslot);
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip) af[set][ip] = *(const uint4*)(buf + SW + (wp * WP + ip * 16) * ROWB + rslot);
    };
    set_tap();
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (p < steps) issue(bufs[p]);
    sync_step(0);
    if (STAGES - 1 < steps) issue(bufs[STAGES - 1]);
    rd(0, bufs[0]);
    static_assert(STAGES % 2 == 0, "register sets alternate with the stage buffers");
    auto mfma = [&](int set) {
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip)
#pragma unroll
        for (int ic = 0; ic < TCN; ++ic) Mma<T>::run(acc[ic][ip], wf[set][ic], af[set][ip]);
    };
    // each step: barrier of s + 1 and the refill, then the reads of s + 1 and the MFMAs of s
    // in one basic block, one read between groups of MFMAs. The last step reads a stale
    // buffer into the idle set (no DMA is in flight by then) so that its block is the same.
    for (int sb = 0; sb < steps; sb += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) {
        const int s = sb + u, cur = u & 1;
        if (s < steps) {
          if (s + 1 < steps) {
            sync_step(s + 1);
            if (s + STAGES < steps) issue(bufs[u]);
          }
          __builtin_amdgcn_sched_barrier(0);
          rd(cur ^ 1, bufs[(u + 1) % STAGES]);
          mfma(cur);
#pragma unroll
          for (int g = 0; g < TCN + TPN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, (TCN * TPN) / (TCN + TPN), 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  } else {
    constexpr int H = TPN / 2;  // the step's MFMAs run in two halves of position fragments
    static_assert(TPN % 2 == 0, "two halves");
    uint4 wf[TCN], af[TPN], an[H];
    auto read_w = [&](const char* buf) {
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) wf[ic] = *(const uint4*)(buf + (wc * WC + ic * 16) * ROWB + rslot);
    };
    auto read_a = [&](const char* buf, int ip0, uint4* dst) {
#pragma unroll
      for (int k = 0; k < H; ++k) dst[k] = *(const uint4*)(buf + SW + (wp * WP + (ip0 + k) * 16) * ROWB + rslot);
    };
    auto mfma_half = [&](int ip0) {
#pragma unroll
      for (int k = 0; k < H; ++k)
#pragma unroll
        for (int ic = 0; ic < TCN; ++ic) Mma<T>::run(acc[ic][ip0 + k], wf[ic], af[ip0 + k]);
    };
    // Two waves per SIMD. The barrier of step s+1 sits between the two halves of step s's
    // MFMAs, so the barrier and the first LDS reads of step s+1 overlap the second half.
    // After the barrier of step k, the DMA of step k + STAGES - 1 refills the buffer of step
    // k - 1, whose reads every wave has completed.
    set_tap();
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (p < steps) issue(bufs[p]);
    sync_step(0);
    if (STAGES - 1 < steps) issue(bufs[STAGES - 1]);
    read_w(bufs[0]);
    read_a(bufs[0], 0, af);
    read_a(bufs[0], H, af + H);
    for (int sb = 0; sb < steps; sb += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) {
        const int s = sb + u;
        if (s < steps) {
          mfma_half(0);
          __builtin_amdgcn_sched_barrier(0);
          const bool more = s + 1 < steps;
          if (more) {
            sync_step(s + 1);
            if (s + STAGES < steps) issue(bufs[u]);
            read_a(bufs[(u + 1) % STAGES], 0, an);
          }
          __builtin_amdgcn_sched_barrier(0);
          mfma_half(H);
          __builtin_amdgcn_sched_barrier(0);
          if (more) {
            read_w(bufs[(u + 1) % STAGES]);
            read_a(bufs[(u + 1) % STAGES], H, af + H);
#pragma unroll
            for (int k = 0; k < H; ++k) af[k] = an[k];
          }
        }
      }
    }
  }

  if (a.ksplit > 1) {
    // split K: the raw float32 sums of this K range go to the partials buffer
    // [ksplit][M][Cout]; k_splitk_reduce adds the ranges in order and runs the epilogue
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) {
      const int m = m0 + wp * WP + ip * 16 + (lane & 15);
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) {
        const int c = c0 + wc * WC + ic * 16 + 4 * (lane >> 4);
        if (m < M && c < a.Cout)
          *(float4*)(a.part + ((int64_t)kz * M + m) * a.Cout + c) =
              make_float4(acc[ic][ip][0], acc[ic][ip][1], acc[ic][ip][2], acc[ic][ip][3]);
      }
    }
    return;
  }
  if (ES == 4 || a.mode == kEpiFramesF32) {
    // fp32, or a bf16 conv with a float32 output: each lane finishes its own 4 channels of
    // each position (conv_epilogue: every mode)
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) {
      const int m = m0 + wp * WP + ip * 16 + (lane & 15);
      if (m >= M) continue;
      const int x = m % a.Wo;
      int q = m / a.Wo;
      const int y = q % a.Ho;
      q /= a.Ho;
      const int b = q % a.B, t = q / a.B;
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) {
        const int c = c0 + wc * WC + ic * 16 + 4 * (lane >> 4);
        if (c >= a.Cout) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[ic][ip][e] + (c + e < a.Cout ? a.bias[c + e] : 0.f);
        conv_epilogue<T>(a, t, b, y, x, c, v);
      }
    }
    return;
  }
  // Epilogue through LDS. Each lane rounds acc + bias to bf16 and writes its 4 channels of
  // one position into the C tile held in the (now idle) stage buffers: rows are positions of
  // TC channels, 8-byte slots permuted by slot ^ (row & 15) so the 16 positions of a fragment
  // hit distinct banks. Then all threads finish 8-channel units (16-byte coalesced reads of
  // the residual and stores of the result).
  constexpr int RB = TC * 2;
  constexpr int RPA = STAGE / RB;
  constexpr int SWZ = TC / 4 - 1 < 15 ? TC / 4 - 1 : 15;  // slot permutation mask
  static_assert(RPA * STAGES >= TP, "the C tile must fit the stage buffers");
  auto crow = [&](int r) -> char* {
    char* base = r < RPA ? s0 : (r < 2 * RPA ? s1 : (r < 3 * RPA ? s2 : s3));
    return base + (r % RPA) * RB;
  };
  __syncthreads();
#pragma unroll
  for (int ip = 0; ip < TPN; ++ip) {
    const int p = wp * WP + ip * 16 + (lane & 15);
    char* row = crow(p);
#pragma unroll
    for (int ic = 0; ic < TCN; ++ic) {
      const int c = wc * WC + ic * 16 + 4 * (lane >> 4);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[ic][ip][e] + (c0 + c + e < a.Cout ? a.bias[c0 + c + e] : 0.f);
      uint2 pk;
      pk.x = pack2_bf16(v[0], v[1]);
      pk.y = pack2_bf16(v[2], v[3]);
      *(uint2*)(row + (((c >> 2) ^ (p & SWZ)) << 3)) = pk;
    }
  }
  __syncthreads();
  if (a.mode == kEpiVideo) {
    // unpatchify + clamp, 4 channels per unit (Cout is not a multiple of 8 here)
    constexpr int UPR4 = TC / 4;
    for (int u = tid; u < TP * UPR4; u += 64 * NWAVE) {
      const int p = u / UPR4, cu = u % UPR4;
      const int m = m0 + p, c = c0 + cu * 4;
      if (m >= M || c >= a.Cout) continue;
      const uint2 w2 = *(const uint2*)(crow(p) + ((cu ^ (p & SWZ)) << 3));
      float v[4] = {bf2f(w2.x & 0xffff), bf2f(w2.x >> 16), bf2f(w2.y & 0xffff), bf2f(w2.y >> 16)};
      const int x = m % a.Wo;
      int q = m / a.Wo;
      const int y = q % a.Ho;
      q /= a.Ho;
      const int b = q % a.B, t = q / a.B;
      conv_epilogue<T>(a, t, b, y, x, c, v);
    }
    return;
  }
  // units: 8 channels of one position; a thread's units step through the positions by
  // PSTEP, so (t, b, y, x) is decoded once and then advanced
  constexpr int UPR = TC / 8;
  constexpr int NT = 64 * NWAVE;
  static_assert(NT % UPR == 0, "units per row must divide the workgroup");
  constexpr int PSTEP = NT / UPR;
  const int cu = tid % UPR, c = c0 + cu * 8;
  int p = tid / UPR;
  int m = m0 + p;
  int x = m % a.Wo, q = m / a.Wo;
  int y = q % a.Ho;
  q /= a.Ho;
  int b = q % a.B, t = q / a.B;
  for (; p < TP && m < M; p += PSTEP, m += PSTEP) {
    if (c < a.Cout) {
      const char* row = crow(p);
      const uint2 lo = *(const uint2*)(row + (((2 * cu) ^ (p & SWZ)) << 3));
      const uint2 hi = *(const uint2*)(row + (((2 * cu + 1) ^ (p & SWZ)) << 3));
      float v[8];
      unpack8_bf16(make_uint4(lo.x, lo.y, hi.x, hi.y), v);
      epilogue8_bf16(a, t, b, y, x, c, v);
    }
    x += PSTEP;
    while (x >= a.Wo) {
      x -= a.Wo;
      if (++y == a.Ho) {
        y = 0;
        if (++b == a.B) {
          b = 0;
          ++t;
        }
      }
    }
  }
}

// Split-K finish: out = epilogue(R(sum over the K ranges, in order, + bias)), one thread per
// 8 channels of one position. The same rounding points as the one-pass epilogue.
__global__ void __launch_bounds__(256) k_splitk_reduce(const ConvArgs a) {
  const int UPR = a.Cout / 8;
  const int64_t M = (int64_t)a.F * a.B * a.Ho * a.Wo;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= M * UPR) return;
  const int64_t m = u / UPR;
  const int c = (int)(u - m * UPR) * 8;
  float v[8];
  const float4 b0 = *(const float4*)(a.bias + c), b1 = *(const float4*)(a.bias + c + 4);
  float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < a.ksplit; ++z) {
    const float* p = a.part + ((int64_t)z * M + m) * a.Cout + c;
    const float4 x0 = *(const float4*)p, x1 = *(const float4*)(p + 4);
    s8[0] += x0.x, s8[1] += x0.y, s8[2] += x0.z, s8[3] += x0.w;
    s8[4] += x1.x, s8[5] += x1.y, s8[6] += x1.z, s8[7] += x1.w;
  }
  const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  const int x = (int)(m % a.Wo);
  int64_t q = m / a.Wo;
  const int y = (int)(q % a.Ho);
  q /= a.Ho;
  const int b = (int)(q % a.B), t = (int)(q / a.B);
  if (a.mode == kEpiFramesF32) {
    float* o = (float*)a.out[t] + b * a.out_bs[t] + ((int64_t)y * a.Wo + x) * a.outC + c;
    *(float4*)o = make_float4(s8[0] + bb[0], s8[1] + bb[1], s8[2] + bb[2], s8[3] + bb[3]);
    *(float4*)(o + 4) = make_float4(s8[4] + bb[4], s8[5] + bb[5], s8[6] + bb[6], s8[7] + bb[7]);
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = bf2f(f2bf(s8[e] + bb[e]));
  epilogue8_bf16(a, t, b, y, x, c, v);
}

// ------------------------------------------------------------------ 3x3 conv with a halo tile (bf16)
//
// For the kh = kw = 3 convs the workgroup owns a 2-D block of TPY x TPX output positions of
// one frame and TC output channels. For each (time tap, 32-channel block) it copies the input
// patch under the block, with its one-pixel border, into LDS once (direct-to-LDS loads); the
// nine spatial taps then read shifted windows of that patch, so the input passes the address
// units once per patch instead of once per tap. Only the weight tile (TC rows of one tap)
// streams per step, through a ring of nine LDS buffers (one per spatial tap). With UP the conv
// reads the nearest x2 upsampling of its input: the patch is the low-resolution region and
// two neighbouring output positions read the same pixel.
//
// Patch pixels are 64-byte rows of 4 chunks stored at slot chunk ^ ((column >> 1) & 3). A
// 16-byte LDS read is served 8 lanes at a time over 128 bytes of banks: with an even patch
// width, 8 consecutive columns fill those banks exactly, for any column shift, and a shift
// by whole patch rows keeps the permutation, so every fragment address is a per-lane base
// (one per column shift and 16-column group) plus a compile-time offset.

// a wave-uniform pointer held in scalar registers (buffer descriptors must be scalar)
__device__ __forceinline__ const char* scalar_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// 16 bytes per lane from base + voff + soff into LDS at lds + 16 * lane (buffer load with
// an LDS destination): a lane whose voff + soff is not below `bytes` receives zeros.
__device__ __forceinline__ void buffer_lds16(const char* base, uint32_t bytes, char* lds, uint32_t voff, int soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(lds), 16, voff, soff, 0, 0);
}

// Patch row (relative to a wave's first) that tile row k reads at tap row dy: the same row
// shifted by dy, or, for the 2x upsampled input, the source row of the nearest neighbour.
template <bool UP>
__host__ __device__ constexpr int halo_rowc(int k, int dy) {
  return UP ? ((k + dy - 1) >> 1) + 1 : k + dy;
}
// The first tap row that reads patch row q (3: none) with RW tile rows per wave.
template <bool UP, int RW>
__host__ __device__ constexpr int halo_first_dy(int q) {
  for (int dy = 0; dy < 3; ++dy)
    for (int k = 0; k < RW; ++k)
      if (halo_rowc<UP>(k, dy) == q) return dy;
  return 3;
}
// How many patch rows are first read at tap row dy.
template <bool UP, int RW>
__host__ __device__ constexpr int rows_first_used(int dy) {
  int n = 0;
  for (int q = 0; q < (UP ? RW / 2 + 2 : RW + 2); ++q) n += halo_first_dy<UP, RW>(q) == dy ? 1 : 0;
  return n;
}
// Interleaves a step's NRD LDS reads with its NMF MFMAs: one read, then MPR MFMAs, the reads
// early in the step (two MFMAs each, the rest after them) so that they have landed by its
// end: 1-3% faster than spread over the whole step, and 3% faster than all reads first.
template <int NRD, int NMF>
__device__ __forceinline__ void interleave_reads() {
  constexpr int MPR = NMF >= 2 * NRD ? 2 : (NMF + NRD - 1) / NRD;
#pragma unroll
  for (int r = 0; r < NRD; ++r) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
  }
  if constexpr (NMF > MPR * NRD) __builtin_amdgcn_sched_group_barrier(0x008, NMF - MPR * NRD, 0);
}

template <int TC, int TPY, int TPX, int WGC, int WGP, bool UP>
__global__ void __launch_bounds__(64 * WGC * WGP, 1) k_conv_halo(const ConvArgs a) {
  using T = bf16_t;
  constexpr int NWAVE = WGC * WGP, NT = 64 * NWAVE;
  constexpr int TP = TPY * TPX;
  constexpr int WC = TC / WGC, WP = TP / WGP, TCN = WC / 16, TPN = WP / 16;
  constexpr int RW = WP / TPX;  // tile rows per wave
  static_assert(WP % TPX == 0 && TPX % 16 == 0, "each wave holds whole tile rows");
  static_assert(!UP || (RW % 2 == 0 && TPY % 2 == 0), "upsampled rows pair up");
  constexpr int PH = UP ? TPY / 2 + 2 : TPY + 2, PW = UP ? TPX / 2 + 2 : TPX + 2;
  static_assert(PW % 2 == 0, "the bank permutation needs an even patch width");
  constexpr int P = PH * PW;
  constexpr int NPI = (P + 15) / 16;                  // patch DMA instructions (16 pixels each)
  constexpr int NPW = (NPI + NWAVE - 1) / NWAVE;      // per wave (the spare ones load zeros)
  constexpr int RB = TC * 2;                          // epilogue staging row (bf16 channels)
  // a patch buffer also holds a quarter of the C tile for the epilogue
  constexpr int PBUF = NPW * NWAVE * 1024 > TP / 4 * RB ? NPW * NWAVE * 1024 : TP / 4 * RB;
  // weight DMA instructions per wave per step (16 rows each). A tile of fewer than 16 rows
  // per wave (the 16-channel tile of conv_out) has one instruction per wave too: the waves
  // past the tile load zeros into a spare 1 KB slot, so that every wave keeps the same count
  // of loads in flight.
  constexpr bool WSPARE = TC < 16 * NWAVE;
  constexpr int NIW = WSPARE ? 1 : TC / (16 * NWAVE);
  static_assert(WSPARE ? TC == 16 : NIW * 16 * NWAVE == TC, "weight rows per wave");
  constexpr int WBUF = TC * 64 + (WSPARE ? 1024 : 0);
  constexpr int RPA = PBUF / RB;
  static_assert(2 * RPA >= TP / 2, "half the C tile fits the patch buffers");
  __shared__ __attribute__((aligned(1024))) char p0[PBUF];
  __shared__ __attribute__((aligned(1024))) char p1[PBUF];
  __shared__ __attribute__((aligned(1024))) char w0[WBUF];
  __shared__ __attribute__((aligned(1024))) char w1[WBUF];
  __shared__ __attribute__((aligned(1024))) char w2[WBUF];
  __shared__ __attribute__((aligned(1024))) char w3[WBUF];
  __shared__ __attribute__((aligned(1024))) char w4[WBUF];
  __shared__ __attribute__((aligned(1024))) char w5[WBUF];
  __shared__ __attribute__((aligned(1024))) char w6[WBUF];
  __shared__ __attribute__((aligned(1024))) char w7[WBUF];
  __shared__ __attribute__((aligned(1024))) char w8[WBUF];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nct = (a.Cout + TC - 1) / TC;
  const int tiles_x = (a.Wo + TPX - 1) / TPX, tiles_y = (a.Ho + TPY - 1) / TPY;
  // block coordinates are wave-uniform: keep them scalar so that the frame tables are read
  // with scalar loads
  // split K: workgroup range kz of a.ksplit takes the kz-th contiguous range of step groups
  const int ntiles = nct * tiles_x * tiles_y * a.F * a.B;
  const int bid0 = xcd_remap(blockIdx.x, gridDim.x);
  const int kz = __builtin_amdgcn_readfirstlane(bid0 / ntiles);
  const int bid = bid0 - kz * ntiles;
  const int ct = __builtin_amdgcn_readfirstlane(bid % nct);
  int rem = __builtin_amdgcn_readfirstlane(bid / nct);
  const int tx = __builtin_amdgcn_readfirstlane(rem % tiles_x);
  rem = __builtin_amdgcn_readfirstlane(rem / tiles_x);
  const int ty = __builtin_amdgcn_readfirstlane(rem % tiles_y);
  rem = __builtin_amdgcn_readfirstlane(rem / tiles_y);
  const int b = __builtin_amdgcn_readfirstlane(rem % a.B), t = __builtin_amdgcn_readfirstlane(rem / a.B);
  const int c0 = ct * TC, Y0 = ty * TPY, X0 = tx * TPX;
  const int csteps = a.Cin / 32;
  // step groups: (time tap, channel block), nine spatial taps each; this workgroup's range
  const int G_all = a.kt * csteps;
  const int g_begin = (int)((int64_t)G_all * kz / a.ksplit);
  const int G = (int)((int64_t)G_all * (kz + 1) / a.ksplit) - g_begin;
  const int S = 9 * G;
  const int64_t Ktot = (int64_t)a.kt * 9 * a.Cin;
  const char* zero = (const char*)g_zero_page;
  const int lrow = lane >> 2, lslot = lane & 3;

  // The copies are buffer loads into LDS: a 32-bit per-lane offset against a descriptor in
  // scalar registers. A lane whose offset is past the descriptor's size receives zeros (the
  // padding around the frame, a missing history frame).
  const int Cin = a.Cin, kt = a.kt;
  constexpr uint32_t kOut = 0x80000000u;  // offset beyond every descriptor: zeros
  // weight DMA: as in k_conv_dma (rows of 64 bytes, slot = chunk ^ ((row >> 1) & 3))
  const int lchunk = lslot ^ ((lrow >> 1) & 3);
  // rows past Cout lie past the descriptor's size and read as zeros
  const char* wbase = scalar_ptr((const T*)a.w + (int64_t)c0 * Ktot);
  const uint32_t wbytes = (uint32_t)((a.Cout - c0 < TC ? a.Cout - c0 : TC) * Ktot * 2);
  uint32_t woffl[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) woffl[i] = (uint32_t)((((wave * NIW + i) * 16 + lrow) * Ktot + lchunk * 8) * 2);
  // the LDS row of a wave's weight instruction (the spare slot for the waves past the tile)
  auto wdst = [&](int i) { return WSPARE && wave > 0 ? TC * 64 : (wave * NIW + i) * 1024; };

  // patch DMA: instruction i of this wave fills pixels (i * NWAVE + wave) * 16 + lane / 4
  // (recomputed at each patch issue, once per nine steps, rather than held in registers)
  const int oy = UP ? (Y0 >> 1) - 1 : Y0 - 1, ox = UP ? (X0 >> 1) - 1 : X0 - 1;
  const int Hin = a.Hin, Win = a.Win;
  auto poff = [&](int i) -> uint32_t {
    const int q = (i * NWAVE + wave) * 16 + lrow;
    const int prow = q / PW, pcol = q - prow * PW;
    const int iy = oy + prow, ix = ox + pcol;
    const bool ok = q < P && iy >= 0 && iy < Hin && ix >= 0 && ix < Win;
    return ok ? (uint32_t)(((iy * Win + ix) * Cin + (lslot ^ ((pcol >> 1) & 3)) * 8) * 2) : kOut;
  };
  const uint32_t fbytes = (uint32_t)a.Hin * a.Win * Cin * 2;
  const char* fb0 = nullptr;
  const char* fb1 = nullptr;
  const char* fb2 = nullptr;
  if (a.in[t]) fb0 = scalar_ptr((const T*)a.in[t] + b * a.in_bs[t]);
  if (kt > 1) {
    if (a.in[t + 1]) fb1 = scalar_ptr((const T*)a.in[t + 1] + b * a.in_bs[t + 1]);
    if (a.in[t + 2]) fb2 = scalar_ptr((const T*)a.in[t + 2] + b * a.in_bs[t + 2]);
  }

  // wofs: byte offset of a group's first tap in a weight row; a patch is (frame base, channel
  // byte offset). Groups advance without divisions: channel block minor, time tap major.
  // a step past the last loads zeros (an empty descriptor): every wave issues the same loads
  // at every step, so the wait counts below are constants
  // step j of a group takes tap (dy, dx) = (j % 3, j / 3), stored at tap index 3 dy + dx
  auto issue_w = [&](char* buf, int wofs, int j, bool valid) {
    const int so = wofs + ((j % 3) * 3 + j / 3) * Cin * 2;
    const uint32_t nb = valid && !(WSPARE && wave > 0) ? wbytes : 0u;
#pragma unroll
    for (int i = 0; i < NIW; ++i) buffer_lds16(wbase, nb, buf + wdst(i), woffl[i], so);
  };
  // a null base (a missing history frame, or past the last group) loads zeros, so that every
  // wave keeps the same count of loads in flight
  auto issue_p = [&](char* buf, const char* base, int cb2) {
    const char* pbase = scalar_ptr(base != nullptr ? base + cb2 : zero);
    const uint32_t pbytes = base != nullptr ? fbytes : 0u;
#pragma unroll
    for (int i = 0; i < NPW; ++i) buffer_lds16(pbase, pbytes, buf + (i * NWAVE + wave) * 1024, poff(i), 0);
  };
  // cursors over the step groups (channel block minor, time tap major), advanced without
  // divisions: (dt1, cb1) names the group after the current one, (dt2, cb2) the one after that
  const int dt0 = g_begin / csteps, cb0 = (g_begin - dt0 * csteps) * 32;  // the range's first group
  int dt1 = dt0, cb1 = cb0, dt2 = dt0, cb2 = cb0;
  const char* fb2p = fb0;
  auto step_group = [&](int& dt, int& cb) {
    cb += 32;
    if (cb == Cin) {
      cb = 0;
      ++dt;
    }
  };
  auto frame_of = [&](int dt) -> const char* { return dt == 0 ? fb0 : (dt == 1 ? fb1 : (dt == 2 ? fb2 : nullptr)); };
  step_group(dt1, cb1);
  step_group(dt2, cb2);
  step_group(dt2, cb2);
  fb2p = frame_of(dt2);

  const int wc = wave / WGP, wp = wave % WGP;
  f32x4_t acc[TCN][TPN];
#pragma unroll
  for (int ic = 0; ic < TCN; ++ic)
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) acc[ic][ip] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // weight fragments: row base + (lane & 15), logical chunk lane >> 4
  const int wrd = (wc * WC + (lane & 15)) * 64 + ((lane >> 4) ^ (((lane & 15) >> 1) & 3)) * 16;
  // patch fragment bases, per 16-column group and column shift dx
  constexpr int NXG = TPX / 16;
  int pvb[NXG][3];
#pragma unroll
  for (int xg = 0; xg < NXG; ++xg)
#pragma unroll
    for (int dx = 0; dx < 3; ++dx) {
      const int px = xg * 16 + (lane & 15);
      const int col = UP ? ((px + dx - 1) >> 1) + 1 : px + dx;
      const int wrow = UP ? wp * (RW / 2) : wp * RW;
      pvb[xg][dx] = (wrow * PW + col) * 64 + (((lane >> 4) ^ ((col >> 1) & 3)) << 4);
    }

  // Taps run dx-major: step j of a group is tap (dy, dx) = (j % 3, j / 3), so the three steps
  // of one column shift dx read the same patch rows shifted by one row each. A patch row's
  // fragments are read once per dx and kept in registers for every dy that uses them: tile row
  // k with tap dy reads patch row rowc(k, dy), so a column shift reads the RW + 2 rows
  // (RW / 2 + 2 upsampled) once instead of 3 RW times. The rows the first step of a column
  // shift needs are read during the last step of the one before; the rest one step before
  // their first use. Weight fragments: two register sets, step s computes from set s & 1
  // while step s + 1's are read into the other.
  constexpr int NQ = UP ? RW / 2 + 2 : RW + 2;  // patch rows a column shift reads
  uint4 wf[2][TCN], bc[NQ][NXG];
  auto read_w = [&](int set, const char* wbuf) {
#pragma unroll
    for (int ic = 0; ic < TCN; ++ic) wf[set][ic] = *(const uint4*)(wbuf + wrd + ic * 16 * 64);
  };
  // the rows q of column shift dx whose first use is at tap row dy0
  auto read_rows = [&](const char* pbuf, int dx, int dy0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (halo_first_dy<UP, RW>(q) == dy0)
#pragma unroll
        for (int xg = 0; xg < NXG; ++xg) bc[q][xg] = *(const uint4*)(pbuf + pvb[xg][dx] + q * PW * 64);
  };
  auto mfma_all = [&](int set, int dy) {
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip)
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) Mma<T>::run(acc[ic][ip], wf[set][ic], bc[halo_rowc<UP>(ip / NXG, dy)][ip % NXG]);
  };
  // waits until this wave's loads of step x (and, at a group's first step, the group's patch,
  // issued before them) have landed and its LDS reads have returned, then the barrier. After
  // W(x) each wave has issued W(x + 1) .. W(x + 7), and the next group's patch when x is not
  // a group's first step.
  auto sync_step = [&](int jx) {
    if (jx == 0)
      wait_vm_lgkm0<7 * NIW>();
    else
      wait_vm_lgkm0<7 * NIW + NPW>();
    __builtin_amdgcn_s_barrier();
  };

  // Pipeline. W(x) (the weight tile of step x) goes to buffer x % 9 at the barrier of step
  // x - 8; the patch of group g + 1 goes to the other patch buffer at the barrier of the
  // group's first step. Step s begins with the barrier of step s + 1: step s's fragments are
  // already in registers, so no wave reads step s's weight buffer nor the previous group's
  // patch any more (the last step of a group reads only the next group's patch), and step
  // s + 1's weight fragments are read into the other register set between step s's MFMAs.
  char* wb[9] = {w0, w1, w2, w3, w4, w5, w6, w7, w8};
  const int wofs0 = (dt0 * 9 * Cin + cb0) * 2;
  issue_p(p0, frame_of(dt0), cb0 * 2);
#pragma unroll
  for (int j = 0; j < 8; ++j) issue_w(wb[j], wofs0, j, true);
  sync_step(0);
  issue_w(wb[8], wofs0, 8, true);
  issue_p(p1, frame_of(dt1), cb1 * 2);
  __builtin_amdgcn_sched_barrier(0);
  read_w(0, wb[0]);
  read_rows(p0, 0, 0);

  int wofs1 = (dt1 * 9 * Cin + cb1) * 2;  // weight offset of the next group
  for (int g0 = 0; g0 < G; g0 += 2) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = g0 + gg;
      if (g < G) {
        char* pcur = gg == 0 ? p0 : p1;
        char* pnext = gg == 0 ? p1 : p0;
        // the last step of all reads finished buffers into registers it leaves unused, so that
        // every step is the same straight-line code
#pragma unroll
        for (int j = 0; j < 9; ++j) {
          const int s = 9 * g + j;
          const int set = (9 * gg + j) & 1;
          const int jn = (j + 1) % 9;
          const int dy = j % 3, dx = j / 3;
          sync_step(jn);
          issue_w(wb[j], wofs1, j, s + 9 < S);
          if (j == 8) issue_p(pcur, fb2p, cb2 * 2);
          __builtin_amdgcn_sched_barrier(0);
          read_w(set ^ 1, wb[jn]);
          mfma_all(set, dy);
          // the patch rows whose first use is the next step: after a column shift's last tap
          // row, the next shift's first rows (from the next group's patch after step 8)
          if (dy == 2)
            read_rows(j == 8 ? pnext : pcur, jn / 3, 0);
          else
            read_rows(pcur, dx, dy + 1);
          // one LDS read between groups of MFMAs, the reads early in the step
          if (dy == 2)
            interleave_reads<TCN + NXG * rows_first_used<UP, RW>(0), TCN * TPN>();
          else if (dy == 0)
            interleave_reads<TCN + NXG * rows_first_used<UP, RW>(1), TCN * TPN>();
          else
            interleave_reads<TCN + NXG * rows_first_used<UP, RW>(2), TCN * TPN>();
          __builtin_amdgcn_sched_barrier(0);
        }
        // the cursors move one group on
        step_group(dt1, cb1);
        wofs1 = (dt1 * 9 * Cin + cb1) * 2;
        step_group(dt2, cb2);
        fb2p = frame_of(dt2);
      }
    }
  }

  wait_vm_lgkm0<0>();
  if (a.ksplit > 1) {
    // split K: the raw float32 sums of this range go to the partials buffer [ksplit][M][Cout]
    // (position m = ((t * B + b) * Ho + y) * Wo + x); k_splitk_reduce finishes them
    const int64_t M = (int64_t)a.F * a.B * a.Ho * a.Wo;
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) {
      const int p = wp * WP + ip * 16 + (lane & 15);
      const int y = Y0 + p / TPX, x = X0 + p % TPX;
      const int64_t m = (((int64_t)t * a.B + b) * a.Ho + y) * a.Wo + x;
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) {
        const int c = c0 + wc * WC + ic * 16 + 4 * (lane >> 4);
        if (y < a.Ho && x < a.Wo && c < a.Cout)
          *(float4*)(a.part + ((int64_t)kz * M + m) * a.Cout + c) =
              make_float4(acc[ic][ip][0], acc[ic][ip][1], acc[ic][ip][2], acc[ic][ip][3]);
      }
    }
    return;
  }
  if (a.mode == kEpiFramesF32) {
    // a float32 output: each lane stores its own 4 channels of each position, sums + bias
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) {
      const int p = wp * WP + ip * 16 + (lane & 15);
      const int y = Y0 + p / TPX, x = X0 + p % TPX;
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) {
        const int c = c0 + wc * WC + ic * 16 + 4 * (lane >> 4);
        if (y < a.Ho && x < a.Wo && c < a.Cout) {
          const float4 bb = *(const float4*)(a.bias + c);
          float v[4] = {acc[ic][ip][0] + bb.x, acc[ic][ip][1] + bb.y, acc[ic][ip][2] + bb.z, acc[ic][ip][3] + bb.w};
          conv_epilogue<T>(a, t, b, y, x, c, v);
        }
      }
    }
    return;
  }
  // Epilogue in two passes of half the positions, staged in the patch buffers (rows of TC
  // bf16 channels, 8-byte slots permuted by slot ^ (row & 15)); 8-channel units are then
  // finished and stored with 16-byte accesses.
  constexpr int SWZ = TC / 4 - 1 < 15 ? TC / 4 - 1 : 15;
  auto crow = [&](int r) -> char* { return r < RPA ? p0 + r * RB : p1 + (r - RPA) * RB; };
  float4 bias[TCN];  // (Cout is a multiple of 4: a lane's 4 channels all exist or all do not)
#pragma unroll
  for (int ic = 0; ic < TCN; ++ic) {
    const int c = c0 + wc * WC + ic * 16 + 4 * (lane >> 4);
    bias[ic] = c < a.Cout ? *(const float4*)(a.bias + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  constexpr int UPR = TC / 8;
  static_assert(NT % UPR == 0, "units per row divide the workgroup");
  constexpr int PSTEP = NT / UPR;
  const int cu = tid % UPR;
  // The residual unit that each 8-channel store adds is copied ahead into the idle weight
  // buffers (unit it of thread tid at buffer it, byte 16 tid; direct-to-LDS loads, one batch
  // per pass issued before the staging) rather than loaded by each store in turn: on the
  // level-3 residual convs 3% faster. (The same for the DupUp3D source was 1% slower.)
  constexpr int NIT = TC == 16 ? 1 : (TP / 2) / PSTEP;
  // (not compiled into the upsampling instances, whose convs add a DupUp3D sum, no residual)
  constexpr bool XPRE = !UP && TC != 16 && NIT <= 9 && NT * 16 <= WBUF;
  static_assert(TC == 16 || NIT * PSTEP == TP / 2, "units per pass divide the threads");
  const bool xres = XPRE && a.mode == kEpiFrames && a.has_res && !a.has_dup;
  char* const wbl[9] = {w0, w1, w2, w3, w4, w5, w6, w7, w8};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
    if constexpr (XPRE) {
      if (xres) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int p = h * (TP / 2) + tid / UPR + it * PSTEP;
          const int y = Y0 + p / TPX, x = X0 + p % TPX;
          const T* src = y < a.Ho && x < a.Wo
                             ? (const T*)a.res[t] + b * a.res_bs[t] + ((int64_t)y * a.Wo + x) * a.outC + c0 + cu * 8
                             : (const T*)g_zero_page;
          __builtin_amdgcn_global_load_lds((const void*)src, LDS_PTR(wbl[it] + wave * 1024), 16, 0, 0);
        }
      }
    }
    if (wp / (WGP / 2) == h) {
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip) {
        const int r = (wp - h * (WGP / 2)) * WP + ip * 16 + (lane & 15);
        char* row = crow(r);
#pragma unroll
        for (int ic = 0; ic < TCN; ++ic) {
          const int c = wc * WC + ic * 16 + 4 * (lane >> 4);
          uint2 pk;
          pk.x = pack2_bf16(acc[ic][ip][0] + bias[ic].x, acc[ic][ip][1] + bias[ic].y);
          pk.y = pack2_bf16(acc[ic][ip][2] + bias[ic].z, acc[ic][ip][3] + bias[ic].w);
          *(uint2*)(row + (((c >> 2) ^ (r & SWZ)) << 3)) = pk;
        }
      }
    }
    if constexpr (XPRE) {
      if (xres) wait_vm_lgkm0<0>();  // this wave's copies of the pass have landed
    }
    __syncthreads();
    if constexpr (TC == 16) {
      // conv_out: unpatchify + clamp, 4 channels per unit (Cout is not a multiple of 8 here)
      constexpr int UPR4 = TC / 4;
      for (int u = tid; u < TP / 2 * UPR4; u += NT) {
        const int r = u / UPR4, cu4 = u % UPR4;
        const int p = h * (TP / 2) + r;
        const int y = Y0 + p / TPX, x = X0 + p % TPX, c = c0 + cu4 * 4;
        if (y < a.Ho && x < a.Wo && c < a.Cout) {
          const uint2 w2 = *(const uint2*)(crow(r) + ((cu4 ^ (r & SWZ)) << 3));
          float v[4] = {bf2f(w2.x & 0xffff), bf2f(w2.x >> 16), bf2f(w2.y & 0xffff), bf2f(w2.y >> 16)};
          conv_epilogue<T>(a, t, b, y, x, c, v);
        }
      }
    } else if (XPRE && xres) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int r = tid / UPR + it * PSTEP;
        const int p = h * (TP / 2) + r;
        const int y = Y0 + p / TPX, x = X0 + p % TPX;
        if (y < a.Ho && x < a.Wo) {
          const char* row = crow(r);
          const uint2 lo = *(const uint2*)(row + (((2 * cu) ^ (r & SWZ)) << 3));
          const uint2 hi = *(const uint2*)(row + (((2 * cu + 1) ^ (r & SWZ)) << 3));
          float v[8], r8[8];
          unpack8_bf16(make_uint4(lo.x, lo.y, hi.x, hi.y), v);
          unpack8_bf16(*(const uint4*)(wbl[it] + tid * 16), r8);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = bf2f(f2bf(v[e] + r8[e]));
          st16_nt((T*)a.out[t] + b * a.out_bs[t] + ((int64_t)y * a.Wo + x) * a.outC + c0 + cu * 8, pack8_bf16(v));
        }
      }
    } else {
      for (int r = tid / UPR; r < TP / 2; r += PSTEP) {
        const int p = h * (TP / 2) + r;
        const int y = Y0 + p / TPX, x = X0 + p % TPX;
        if (y < a.Ho && x < a.Wo) {
          const char* row = crow(r);
          const uint2 lo = *(const uint2*)(row + (((2 * cu) ^ (r & SWZ)) << 3));
          const uint2 hi = *(const uint2*)(row + (((2 * cu + 1) ^ (r & SWZ)) << 3));
          float v[8];
          unpack8_bf16(make_uint4(lo.x, lo.y, hi.x, hi.y), v);
          epilogue8_bf16(a, t, b, y, x, c0 + cu * 8, v);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ RMS norm (+ SiLU)
//
// y = x / max(||x||_2, 1e-12) (rounded), * sqrt(C) (rounded), * gamma (rounded), then
// optionally SiLU (rounded): the 16-bit chain of the page's "Precision" section; in fp32
// every rounding is the float32 one.

// SiLU u / (1 + exp(-u)) of a bf16 value u to about one float32 ulp in a few instructions.
// exp(-u) = 2^(-u L) e^(u (L - log2 e) ln 2) with L = log2(e) to 16 significant bits: the
// product -u L of the 8-bit u is exact in float32, the hardware 2^x takes it, and the small
// remainder factor is 1 + a (a = u (L - log2 e) ln 2, |a| < 1e-4 for |u| < 16). The quotient
// comes from the hardware reciprocal with one Newton correction. Where exp(-u) overflows
// (u < -88) the quotient is -0, the limit.
__device__ __forceinline__ float silu_bf16(float u) {
  constexpr float kL16 = 1.44268798828125f;      // 47274 / 2^15
  constexpr float kRem = -4.8884954e-06f;        // (kL16 - log2 e) ln 2
  const float E = __builtin_amdgcn_exp2f(-u * kL16);
  const float e = __builtin_fmaf(E, u * kRem, E);
  const float d = 1.f + e;
  const float r = __builtin_amdgcn_rcpf(d);
  const float q0 = u * r;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, d, u), r, q0);
  return d < 3.0e38f ? q : -0.f;
}

// One wave per position, C <= 1024 (the widths without a k_norm_v instance).
template <typename T>
__global__ void __launch_bounds__(256) k_norm(const NormArgs a) {
  using X = Elem<T>;
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t M = (int64_t)a.F * a.B * a.HW;
  if (m >= M) return;
  const int pos = (int)(m % a.HW);
  const int64_t q = m / a.HW;
  const int b = (int)(q % a.B), t = (int)(q / a.B);
  const T* x = (const T*)a.in[t] + b * a.in_bs[t] + (int64_t)pos * a.C;
  T* y = (T*)a.out[t] + b * a.out_bs[t] + (int64_t)pos * a.C;
  float v[16];
  // the sum of squares and the normalisation in float64 for bf16 (as in k_norm_v)
  using Acc = typename std::conditional<sizeof(T) == 2, double, float>::type;
  Acc ss = 0;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = (it * 64 + lane) * 4;
    if (c < a.C) {
      X::ld4(x + c, v + 4 * it);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += (Acc)v[4 * it + e] * (Acc)v[4 * it + e];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const Acc d = ss > (Acc)1e-24 ? (Acc)sqrt(ss) : (Acc)1e-12;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = (it * 64 + lane) * 4;
    if (c < a.C) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float u = X::R((float)((Acc)v[4 * it + e] / d));
        u = X::R(u * a.sqrtC);
        u = X::R(u * a.gamma[c + e]);
        if (a.silu) u = X::R(sizeof(T) == 2 ? silu_bf16(u) : u / (1.f + expf(-u)));
        o[e] = u;
      }
      X::st4(y + c, o);
    }
  }
}

// SiLU of the bf16 values u = 0 and 2^-16 <= |u| < 2^16 (but the largest binade's last
// value), as a table of bf16 results held in LDS: per sign s, entry (s << 12) | 0 for zero and
// (s << 12) | (|u| bits - kSiluLo + 1) for the others. Each entry is silu_bf16 of its value
// rounded to bf16 (round to nearest even), the very result the arithmetic path stores, so a
// lookup and the arithmetic agree bit for bit. Other values (0 < |u| < 2^-16, the largest,
// inf, NaN) take the arithmetic path. Zero has its own entries because exact zeros are common
// (a bf16 sum of two opposite values): |u| bits m give the entry max(m - kSiluLo + 1, 0),
// which is 0 for zero and for the small values, and m - 1 < kSiluLo - 1 flags the small
// nonzero ones.
constexpr uint32_t kSiluLo = (127u - 16u) << 7;  // the magnitude bits of 2^-16
constexpr int kSiluSpan = 4096;                   // zero, then 4,095 magnitudes from 2^-16 on
constexpr int kSiluEntries = 2 * kSiluSpan;       // both signs: 16 KB

// Bandwidth-oriented version: a position's C channels are spread over LPP lanes, each lane
// holding VPL 16-byte vectors; a wave covers 64 / LPP positions per round and R rounds, all
// loads issued before the sums are reduced (xor shuffles within the LPP lanes). bf16 rounds
// two values per conversion instruction, and the last rounding is the packing store's.
// A block is the NWV waves of a workgroup, NWV * PPW * R positions of one frame.
// TAB (bf16 with SiLU): the workgroup first fills the SiLU table in LDS, then walks the
// blocks of every frame with a grid stride (two workgroups of 16 waves per CU, so the table is
// built twice per CU and serves many blocks); without TAB, one block per workgroup and grid
// y = (frame, batch).
template <typename T, int LPP, int VPL, int R, bool SILU, bool TAB = false, int NWV = 4>
__global__ void __launch_bounds__(64 * NWV) k_norm_v(const NormArgs a) {
  using X = Elem<T>;
  constexpr int EV = 16 / (int)sizeof(T);  // elements per 16-byte vector
  constexpr int PPW = 64 / LPP;
  constexpr int CC = LPP * VPL * EV;  // channels of a position
  constexpr bool kSqrtPow2 = CC == 16 || CC == 64 || CC == 256 || CC == 1024;
  static_assert(!TAB || (sizeof(T) == 2 && SILU), "the table holds bf16 SiLU results");
  __shared__ uint16_t tab[TAB ? kSiluEntries : 1];
  const int lane = threadIdx.x & 63, li = lane % LPP;
  if constexpr (TAB) {
    for (int i = threadIdx.x; i < kSiluEntries; i += 64 * NWV) {
      const uint32_t j = (uint32_t)(i & (kSiluSpan - 1));
      const uint32_t h = ((uint32_t)(i >> 12) << 15) | (j ? kSiluLo + j - 1 : 0u);
      tab[i] = f2bf(silu_bf16(__uint_as_float(h << 16)));
    }
    __syncthreads();
  }
  // this lane's gamma values (its channels are the same in every round)
  float g[VPL][EV];
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int e = 0; e < EV; e += 4) {
      const float4 q = *(const float4*)(a.gamma + (v * LPP + li) * EV + e);
      g[v][e] = q.x, g[v][e + 1] = q.y, g[v][e + 2] = q.z, g[v][e + 3] = q.w;
    }
  constexpr int PB = NWV * PPW * R;  // positions per block
  const int nblk = (a.HW + PB - 1) / PB;
  const int nall = TAB ? nblk * a.F * a.B : 1;
  for (int blk = TAB ? (int)blockIdx.x : 0; blk < nall; blk += TAB ? (int)gridDim.x : 1) {
    const int tb = TAB ? blk / nblk : (int)blockIdx.y;
    const int pb = TAB ? blk - tb * nblk : (int)blockIdx.x;
    const int t = tb / a.B, b = tb % a.B;
    const int pos0 = (pb * NWV + (int)(threadIdx.x >> 6)) * PPW * R + lane / LPP;
    const T* xf = (const T*)a.in[t] + b * a.in_bs[t];
    T* yf = (T*)a.out[t] + b * a.out_bs[t];
    uint4 buf[R][VPL];
    T* outp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int pos = pos0 + r * PPW;
      outp[r] = nullptr;
      if (pos < a.HW) {
        const T* x = xf + (int64_t)pos * a.C;
        outp[r] = yf + (int64_t)pos * a.C;
#pragma unroll
        for (int v = 0; v < VPL; ++v) buf[r][v] = *(const uint4*)(x + (v * LPP + li) * EV);
      } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) buf[r][v] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float val[VPL][EV];
      // bf16: the sum of squares in float64, so that ||x|| and x / ||x|| are exact to far below
      // the bf16 rounding that follows; fp32: in float32
      using Acc = typename std::conditional<sizeof(T) == 2, double, float>::type;
      Acc ss = 0;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if constexpr (sizeof(T) == 2) {
          unpack8_bf16(buf[r][v], val[v]);
        } else {
          val[v][0] = __uint_as_float(buf[r][v].x), val[v][1] = __uint_as_float(buf[r][v].y);
          val[v][2] = __uint_as_float(buf[r][v].z), val[v][3] = __uint_as_float(buf[r][v].w);
        }
#pragma unroll
        for (int e = 0; e < EV; ++e) ss += (Acc)val[v][e] * (Acc)val[v][e];
      }
#pragma unroll
      for (int off = LPP / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
      if (!outp[r]) continue;
      const float d = fmaxf(sqrtf((float)ss), 1e-12f);
      // bf16: 1 / max(||x||, 1e-12) in float64, carried as two floats ih + il
      const double dinv = fmin(rsqrt((double)ss), 1e12);
      const float ih = (float)dinv, il = (float)(dinv - (double)ih);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int c0 = (v * LPP + li) * EV;
        float o[EV];
        if constexpr (sizeof(T) == 2) {
          // bf16: x / ||x|| as x ih + x il, rounded once (to within 2^-47 of the float64
          // quotient, then to float32 and bf16, as a float64 value is cast to bf16); the
          // products by sqrt(C) and gamma in float32 (exact before their rounding); SiLU to
          // about one float32 ulp (silu_bf16). A float32 result then lands on the far side of a
          // bf16 rounding boundary from the exact value only where it lies within about an ulp
          // of that boundary.
          auto round2 = [](float& p, float& q) {
            const uint32_t w = pack2_bf16(p, q);
            p = __uint_as_float(w << 16);
            q = __uint_as_float(w & 0xffff0000u);
          };
          if constexpr (TAB) {
            // R(u gamma) for the vector's EV values, packed; then one table read per value
            // when every value of this lane's vector is in the table's range
            uint32_t w[EV / 2];
            uint32_t hi_m = 0, lo_m1 = 0xffffffffu;  // max entry offset, min (|u| bits - 1)
            uint32_t ia[EV];
#pragma unroll
            for (int e = 0; e < EV; e += 2) {
              float u0 = __builtin_fmaf(val[v][e], ih, val[v][e] * il);
              float u1 = __builtin_fmaf(val[v][e + 1], ih, val[v][e + 1] * il);
              round2(u0, u1);
              u0 *= a.sqrtC, u1 *= a.sqrtC;
              if constexpr (!kSqrtPow2) round2(u0, u1);
              w[e / 2] = pack2_bf16(u0 * g[v][e], u1 * g[v][e + 1]);
#pragma unroll
              for (int k = 0; k < 2; ++k) {
                const uint32_t h = k ? w[e / 2] >> 16 : w[e / 2] & 0xffffu;
                const uint32_t mag = h & 0x7fffu;
                const uint32_t m = mag > kSiluLo - 1u ? mag - (kSiluLo - 1u) : 0u;
                hi_m = max(hi_m, m);
                lo_m1 = min(lo_m1, mag - 1u);     // zero wraps to the top
                ia[e + k] = ((h >> 15) << 12) | m;  // read only when every m is below the span
              }
            }
            uint4 res;
            uint32_t* rw = (uint32_t*)&res;
            if (hi_m < (uint32_t)kSiluSpan && lo_m1 >= kSiluLo - 1u) {
#pragma unroll
              for (int e = 0; e < EV; e += 2) rw[e / 2] = (uint32_t)tab[ia[e]] | ((uint32_t)tab[ia[e + 1]] << 16);
            } else {
#pragma unroll
              for (int e = 0; e < EV; ++e) o[e] = silu_bf16(__uint_as_float(e & 1 ? w[e / 2] & 0xffff0000u : w[e / 2] << 16));
              res = pack8_bf16(o);
            }
            *(uint4*)(outp[r] + c0) = res;
            continue;
          } else {
#pragma unroll
            for (int e = 0; e < EV; e += 2) {
              float u0 = __builtin_fmaf(val[v][e], ih, val[v][e] * il);
              float u1 = __builtin_fmaf(val[v][e + 1], ih, val[v][e + 1] * il);
              round2(u0, u1);
              u0 *= a.sqrtC, u1 *= a.sqrtC;
              // C = 16, 64, 256, 1024: sqrt(C) is a power of two, the product exact, its
              // rounding the identity
              if constexpr (!kSqrtPow2) round2(u0, u1);
              u0 *= g[v][e], u1 *= g[v][e + 1];
              if constexpr (SILU) {
                round2(u0, u1);
                u0 = silu_bf16(u0);
                u1 = silu_bf16(u1);
              }
              o[e] = u0, o[e + 1] = u1;  // rounded by the packing store
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < EV; ++e) {
            float u = val[v][e] / d;
            u = u * a.sqrtC;
            u = u * g[v][e];
            if constexpr (SILU) u = u / (1.f + expf(-u));
            o[e] = u;
          }
        }
        if constexpr (sizeof(T) == 2) {
          *(uint4*)(outp[r] + c0) = pack8_bf16(o);
        } else {
          *(float4*)(outp[r] + c0) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ attention
//
// Max or sum over each aligned group of N (2, 4, 8 or 16) lanes, every lane getting the
// group's result, with DPP lane moves (no LDS): swaps within pairs and quads, then the
// mirror of each half-row (8 lanes) and of each row (16 lanes). The partners' values are
// combined in one order for the whole group, so every lane holds the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int N, bool MAX>
__device__ __forceinline__ float group_reduce(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1 to 16 lanes");
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (N >= 2) v = op(v, dpp_mov<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) v = op(v, dpp_mov<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) v = op(v, dpp_mov<0x141>(v));  // row_half_mirror
  if constexpr (N >= 16) v = op(v, dpp_mov<0x140>(v)); // row_mirror
  return v;
}
//
// One workgroup: 32 queries (2 tiles of 16) of one frame, NW waves; wave w owns head dims
// [w*DW, (w+1)*DW). Per block of 32 keys each wave computes its partial S^T = K Q^T over its
// dims (MFMA, Q fragments held in registers), the partials are summed through LDS (each
// wave sums 1/NW of the tile over all waves, in wave order, so the result is deterministic;
// then every wave reads the whole sum), then every wave runs the online softmax on
// the full scores and accumulates O^T += V^T P for its own dims. S^T's accumulator layout
// (keys 4g..4g+3 of each 16-key tile in lane group g, one query per lane) is directly the
// k layout of P as the B operand of the PV MFMA; V^T is stored with its keys in that order
// (vt_slot), so a lane's 8 keys of a block are one 16-byte load.
// PF: loads run one phase ahead of their use (bf16, where the registers still allow the
// variant's workgroups per CU: 8 waves, or 4 waves of at most 96 dims); without it each
// block's K and V fragments are loaded right before their products, which leaves the fp32
// variant with C = 1024 and the 4-wave C = 512 one the registers they need.
// RS (8 waves): the summed scores are scattered over the waves and every wave then runs the
// online softmax over the whole tile for itself, after the second barrier, where it
// overlaps the other waves' products. Without RS (fewer waves) each wave finishes the
// softmax of its own query rows and shares P and the rescale factors through LDS.
template <typename T, int NW, int DW, bool PF = (sizeof(T) == 2 && (NW >= 8 || DW <= 96)), bool RS = (NW >= 8)>
__global__ void __launch_bounds__(64 * NW) k_attn(const AttnArgs a) {
  using X = Elem<T>;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KS = BF ? 32 : 16;  // head dims per S MFMA step
  constexpr int NKS = DW / KS;
  constexpr int NDT = DW / 16;       // 16-dim tiles of O per wave
  // softmax rows: wave w finishes queries [w * QPW, (w + 1) * QPW) of the block, LPQ lanes
  // per query, EPL consecutive keys per lane
  constexpr int QPW = 32 / NW, LPQ = 64 / QPW, EPL = 32 / LPQ;
  static_assert(QPW * NW == 32 && LPQ * QPW == 64 && EPL * LPQ == 32, "the tile splits evenly over the lanes");
  constexpr int PR = BF ? 40 : 36;  // P row stride in elements (16-byte aligned, padded)
  // each wave's partial S^T tile: 4 (kt, qt) tiles of 64 accumulator vectors, vector l16 + 16 g
  // at slot l16 + GS g. With RS the tile is dense (the reduce-scatter reads it as 1,024 floats);
  // without, key groups are 18 slots apart and (kt, qt) tiles 76, so that the 16 lanes of two
  // queries' rows (8 (kt, g) each) fall in 16 different 4-bank groups
  constexpr int GS = RS ? 16 : 18, TS = RS ? 64 : 76;
  __shared__ f32x4_t red[2][NW][4][TS];
  __shared__ f32x4_t rsum[2][RS ? 4 : 1][64];  // (RS) the summed tile
  __shared__ __attribute__((aligned(16))) T ptile[2][RS ? 1 : 32][PR];  // P (rounded to T), keys in vt_slot order
  __shared__ float alph[2][RS ? 1 : 32];  // each query's rescale factor of the block
  __shared__ float2 mlq[RS ? 1 : 32];     // each query's final (max, sum)

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  // (query block, frame, key range), query blocks fastest, renumbered so that each XCD runs
  // a contiguous run: its CUs sweep the same frame's (or key range's) K and V together,
  // which its L2 then serves to all of them
  const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int N = xcd_remap(L, gridDim.x * gridDim.y * gridDim.z);
  const int qb = N % gridDim.x, fz = N / gridDim.x;
  const int fr = fz % gridDim.y, q0 = qb * 32;
  // key range of this workgroup: blocks of 32 keys [kb0, kb1) of the frame's ceil(S / 32)
  const int nkb = (a.S + 31) / 32, kz = fz / gridDim.y;
  const int kb0 = (int)((int64_t)nkb * kz / a.ksplit), kb1 = (int)((int64_t)nkb * (kz + 1) / a.ksplit);
  const int C = a.C, S = a.S, Sp = a.Sp;
  const T* Q = (const T*)a.q + (int64_t)fr * S * C;
  const T* K = (const T*)a.k + (int64_t)fr * S * C;
  const T* Vt = (const T*)a.vt + (int64_t)fr * C * Sp;
  const int dw0 = w * DW;
  const float sc = a.scale * 1.4426950408889634f;  // softmax in base 2

  uint4 qf[NKS][2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qi = min(q0 + qt * 16 + l16, S - 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks][qt] = *(const uint4*)(Q + (int64_t)qi * C + dw0 + ks * KS + g * (BF ? 8 : 4));
  }
  f32x4_t o[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt][0] = o[dt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the softmax row this lane finishes: query sq of the block (tile sqt, row sql), keys
  // k0 .. k0 + EPL - 1 of each key block; its running max and sum (the same in the LPQ lanes)
  const int sq = w * QPW + lane / LPQ, sqt = sq >> 4, sql = sq & 15, k0 = (lane % LPQ) * EPL;
  float mrow = -INFINITY, lrow = 0.f;
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};  // (RS) per query tile

  // PF: a block's K fragments are loaded during the block before (behind its reduction,
  // softmax and P V products), and its V fragments (bf16) at the top of the block, ahead
  // of the S products.
  uint4 kf[NKS][2];
  auto load_k = [&](int kv0) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = min(kv0 + kt * 16 + l16, S - 1);
        kf[ks][kt] = *(const uint4*)(K + (int64_t)key * C + dw0 + ks * KS + g * (BF ? 8 : 4));
      }
  };
  if (PF && kb0 < kb1) load_k(kb0 * 32);

  int par = 0;
  for (int kv0 = kb0 * 32; kv0 < kb1 * 32; kv0 += 32, par ^= 1) {
    uint4 vf[BF ? NDT : 1];
    auto load_v = [&]() {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        // keys 4g..4g+3 of both halves of the block: one vector (vt_slot)
        vf[dt] = *(const uint4*)(Vt + (int64_t)(dw0 + dt * 16 + l16) * Sp + kv0 + 8 * g);
      }
    };
    if constexpr (BF && PF) load_v();
    if constexpr (!PF) load_k(kv0);
    f32x4_t s[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt][0] = s[kt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        Mma<T>::run(s[kt][0], kf[ks][kt], qf[ks][0]);
        Mma<T>::run(s[kt][1], kf[ks][kt], qf[ks][1]);
      }
    }
    // (after the last block this loads keys it will not use: kept unconditional, so that the
    // load counts the waits below see are the same on every iteration)
    if constexpr (PF) load_k(kv0 + 32);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) red[par][w][kt * 2 + qt][l16 + GS * g] = s[kt][qt];
    __syncthreads();
    float p[2][2][4];  // (RS, or fp32) key 16 kt + 4 g + e of query 16 qt + l16
    if constexpr (RS) {
      {
        // reduce-scatter: wave w sums floats [w * FPW, (w + 1) * FPW) of the tile over the waves,
        // in wave order, and every wave then reads the whole summed tile
        constexpr int FPW = 1024 / NW, FPL = FPW / 64;
        static_assert(FPL * 64 * NW == 1024, "the tile splits evenly over the waves' lanes");
        const float* rf = (const float*)&red[par][0][0][0];
        float* sf = (float*)&rsum[par][0][0];
        const int f0 = w * FPW + lane * FPL;
        float acc[FPL];
#pragma unroll
        for (int e = 0; e < FPL; ++e) acc[e] = rf[f0 + e];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww)
#pragma unroll
          for (int e = 0; e < FPL; ++e) acc[e] += rf[ww * 1024 + f0 + e];
#pragma unroll
        for (int e = 0; e < FPL; ++e) sf[f0 + e] = acc[e];
      }
      __syncthreads();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) s[kt][qt] = rsum[par][kt * 2 + qt][lane];
      // online softmax; key of element e in tile kt: kv0 + kt*16 + 4g + e
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = kv0 + kt * 16 + 4 * g + e;
            const float v = key < S ? s[kt][qt][e] * sc : -INFINITY;
            p[kt][qt][e] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(mrun[qt], mx);
        const float alpha = exp2f(mrun[qt] - mnew);
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = exp2f(p[kt][qt][e] - mnew);
            p[kt][qt][e] = pe;
            sum += pe;
          }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        lrun[qt] = lrun[qt] * alpha + sum;
        mrun[qt] = mnew;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt][qt] *= alpha;
      }
    } else {
      {
        // each lane sums its EPL scores over the waves' partials, in wave order (deterministic),
        // then the online softmax of its query runs over the query's LPQ lanes; P goes to LDS
        // rounded to T, with the query's rescale factor. Element (key 16 kt + 4 g + e, query
        // 16 qt + l) of a partial is float 4 (TS (2 kt + qt) + l + GS g) + e.
        const float* rf = (const float*)&red[par][0][0][0];
        float v[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int key = k0 + e;
          const int idx = ((((key >> 4) * 2 + sqt) * TS + sql + GS * ((key >> 2) & 3)) << 2) + (key & 3);
          float acc = rf[idx];
#pragma unroll
          for (int ww = 1; ww < NW; ++ww) acc += rf[ww * 16 * TS + idx];
          v[e] = kv0 + key < S ? acc * sc : -INFINITY;
        }
        float mx = v[0];
#pragma unroll
        for (int e = 1; e < EPL; ++e) mx = fmaxf(mx, v[e]);
        mx = group_reduce<LPQ, true>(mx);
        const float mnew = fmaxf(mrow, mx);
        const float alpha = exp2f(mrow - mnew);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          v[e] = exp2f(v[e] - mnew);
          sum += v[e];
        }
        sum = group_reduce<LPQ, false>(sum);
        lrow = lrow * alpha + sum;
        mrow = mnew;
        T* prow = &ptile[par][sq][0];
#pragma unroll
        for (int e = 0; e < EPL; ++e) X::st(prow + vt_slot(k0 + e), v[e]);
        if (lane % LPQ == 0) alph[par][sq] = alpha;
      }
      __syncthreads();
      // O^T[d][q] = alpha_q O^T[d][q] + V^T[d][key] P^T[key][q]; this lane's column is query
      // 16 qt + l16
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float al = alph[par][qt * 16 + l16];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt][qt] *= al;
      }
      if constexpr (!BF) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const float4 pv = *(const float4*)&ptile[par][qt * 16 + l16][8 * g + 4 * kt];
            p[kt][qt][0] = pv.x, p[kt][qt][1] = pv.y, p[kt][qt][2] = pv.z, p[kt][qt][3] = pv.w;
          }
      }
    }
    if constexpr (BF) {
      // P^T's B fragment: keys 4g..4g+3 of both 16-key halves, one vector (vt_slot)
      uint4 pb[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        if constexpr (RS) {
          pb[qt].x = pack2_bf16(p[0][qt][0], p[0][qt][1]);
          pb[qt].y = pack2_bf16(p[0][qt][2], p[0][qt][3]);
          pb[qt].z = pack2_bf16(p[1][qt][0], p[1][qt][1]);
          pb[qt].w = pack2_bf16(p[1][qt][2], p[1][qt][3]);
        } else {
          pb[qt] = *(const uint4*)&ptile[par][qt * 16 + l16][8 * g];
        }
      }
      if constexpr (!PF) load_v();
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        Mma<T>::run(o[dt][0], vf[dt], pb[0]);
        Mma<T>::run(o[dt][1], vf[dt], pb[1]);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const T* vrow = Vt + (int64_t)(dw0 + dt * 16 + l16) * Sp + kv0 + 8 * g;  // (vt_slot)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const float4 vf = *(const float4*)(vrow + kt * 4);
          const float vv[4] = {vf.x, vf.y, vf.z, vf.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[e], p[kt][0][e], o[dt][0], 0, 0, 0);
            o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[e], p[kt][1][e], o[dt][1], 0, 0, 0);
          }
        }
      }
    }
  }
  if constexpr (!RS) {
    // every wave's queries' final (max, sum)
    if (lane % LPQ == 0) mlq[sq] = make_float2(mrow, lrow);
    __syncthreads();
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float2 ml = mlq[qt * 16 + l16];
      mrun[qt] = ml.x, lrun[qt] = ml.y;
    }
  }
  if (a.ksplit > 1) {
    // this key range's unnormalised O and (max, sum): k_attn_combine merges the ranges
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int qi = q0 + qt * 16 + l16;
      if (qi >= S) continue;
      const int64_t row = ((int64_t)kz * a.nfr + fr) * S + qi;
      float* orow = a.opart + row * C + dw0 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *(float4*)(orow + dt * 16) = make_float4(o[dt][qt][0], o[dt][qt][1], o[dt][qt][2], o[dt][qt][3]);
      if (w == 0 && g == 0) *(float2*)(a.ml + row * 2) = make_float2(mrun[qt], lrun[qt]);
    }
    return;
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qi = q0 + qt * 16 + l16;
    if (qi >= S) continue;
    const float inv = 1.f / lrun[qt];
    T* orow = (T*)a.o + ((int64_t)fr * S + qi) * C + dw0 + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[dt][qt][e] * inv;
      X::st4(orow + dt * 16, v);
    }
  }
}

// Key-split finish: O = sum_z 2^(m_z - m) O_z / sum_z 2^(m_z - m) l_z with m = max_z m_z, the
// ranges taken in order; one thread per 4 head dims of one query.
template <typename T>
__global__ void __launch_bounds__(256) k_attn_combine(const AttnArgs a) {
  using X = Elem<T>;
  const int C4 = a.C / 4;
  const int64_t rows = (int64_t)a.nfr * a.S;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= rows * C4) return;
  const int64_t row = u / C4;
  const int d = (int)(u - row * C4) * 4;
  float m = -INFINITY;
  for (int z = 0; z < a.ksplit; ++z) m = fmaxf(m, a.ml[(z * rows + row) * 2]);
  float l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < a.ksplit; ++z) {
    const float2 mlz = *(const float2*)(a.ml + (z * rows + row) * 2);
    const float wz = exp2f(mlz.x - m);
    const float4 oz = *(const float4*)(a.opart + (z * rows + row) * a.C + d);
    l += wz * mlz.y;
    o[0] += wz * oz.x, o[1] += wz * oz.y, o[2] += wz * oz.z, o[3] += wz * oz.w;
  }
  const float inv = 1.f / l;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = o[e] * inv;
  X::st4((T*)a.o + row * a.C + d, v);
}

// ------------------------------------------------------------------ attention, materialised scores (bf16)
//
// The bf16 attention core as two NT GEMMs on MFMA with the scores in between in HBM, so that
// neither GEMM holds a d = C wide accumulator (what limits the flash kernel above to 32
// queries per workgroup at C = 1,024, and so makes it re-read K and V from L2 once per 32
// queries):
//  scores (k_attn_mm<0>): D[j][i] = K_j . Q_i for a tile of keys j x queries i of one frame
//    (K = C). Epilogue: s = D * scale * log2(e); per query and 128-key tile t the max m_t over
//    the tile's keys (keys past S count as -inf); p = 2^(s - m_t) rounded to bf16, stored in
//    P[i][j] with the keys of each 32-key block in the vt_slot order of V^T; l_t = the sum of
//    those rounded p; (m_t, l_t) stored per (query, key tile).
//  k_attn_fac: per query, M = max_t m_t, L = sum_t l_t 2^(m_t - M) and the tile weights
//    f_t = max(2^(m_t - M) / L, 2^-100), written as g_t = f_t / f_t+1 (the last: f_t).
//  P V (k_attn_mm<1>): D[c][i] = sum_t f_t(i) sum_{j in tile t} V^T[c][j] P[i][j] for a tile
//    of channels x queries (K = the frame's keys). After each key tile's products the
//    accumulator is scaled by that tile's g: it then holds (sum_{s <= t} f_s A_s) / f_t+1,
//    at most 2^100 times an output (no overflow), and the last scale leaves sum_t f_t A_t. A
//    tile whose weight is clamped to 2^-100 moves O by under 2^-93 of its scale. O = D
//    rounded to bf16 once: the softmax weights of each query sum to 1 over P's rounded values.
// Both share the pipeline of k_conv_dma: 64-byte rows of 4 chunks (slot = chunk ^ ((row >> 1)
// & 3)), direct-to-LDS loads four steps deep, one barrier per step. Two tile shapes: 128 x 128
// with 4 waves of 64 x 64 and two workgroups per CU, for grids too small to fill the chip
// with larger tiles; 256 x 256 with 8 waves of 128 x 64, half the L2 traffic and a third less
// LDS traffic per FLOP. Rows past the end of a tensor are read from its last row and never
// stored, so every load stays inside the tensor.

template <int MODE, int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN, WGM * WGN == 4 ? 2 : 1) k_attn_mm(const AttnMatArgs a) {
  using T = bf16_t;
  constexpr bool PV = MODE == 1;
  constexpr int NW = WGM * WGN, ROWB = 64, STAGES = 4, KT = 128;
  constexpr int TM = BM / WGM, TN = BN / WGN;  // wave tile
  constexpr int TCN = TM / 16, TPN = TN / 16;  // its 16-row fragments
  constexpr int SA = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int NIA = BM / (16 * NW), NIB = BN / (16 * NW);  // 16-row DMA instructions per wave and step
  constexpr int NI = NIA + NIB;
  constexpr int WPT = KT / TM;  // waves along M per 128-key tile (scores)
  static_assert(NIA * 16 * NW == BM && NIB * 16 * NW == BN && (WPT == 1 || WPT == 2) && TM * WPT == KT,
                "tile / wave split");
  // one array per stage: the compiler then sees that the LDS reads of a step do not alias the
  // copies in flight into the other stages
  __shared__ __attribute__((aligned(1024))) char s0[STAGE];
  __shared__ __attribute__((aligned(1024))) char s1[STAGE];
  __shared__ __attribute__((aligned(1024))) char s2[STAGE];
  __shared__ __attribute__((aligned(1024))) char s3[STAGE];
  char* bufs[STAGES] = {s0, s1, s2, s3};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int S = a.S, Sp = a.Sp, C = a.C;
  const int Mrows = PV ? C : S;  // A rows: channels (P V) or keys (scores)
  const int nmt = (Mrows + BM - 1) / BM, nnt = (S + BN - 1) / BN;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int fr = __builtin_amdgcn_readfirstlane(bid / (nmt * nnt));
  const int rem = bid - fr * nmt * nnt;
  const int nt = __builtin_amdgcn_readfirstlane(rem / nmt), mt = __builtin_amdgcn_readfirstlane(rem - nt * nmt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int lrow = lane >> 2, lslot = lane & 3, lchunk = lslot ^ ((lrow >> 1) & 3);
  const int64_t ld = PV ? Sp : C;  // elements per row of A and of B
  const T* Abase = PV ? (const T*)a.vt + (int64_t)fr * C * Sp : (const T*)a.k + (int64_t)fr * S * C;
  const T* Bbase = PV ? (const T*)a.p + (int64_t)fr * S * Sp : (const T*)a.q + (int64_t)fr * S * C;
  const char* asrc[NIA];
  const char* bsrc[NIB];
#pragma unroll
  for (int i = 0; i < NIA; ++i) {
    const int row = min(m0 + (wave * NIA + i) * 16 + lrow, Mrows - 1);
    asrc[i] = (const char*)(Abase + row * ld) + lchunk * 16;
  }
#pragma unroll
  for (int i = 0; i < NIB; ++i) {
    const int row = min(n0 + (wave * NIB + i) * 16 + lrow, S - 1);
    bsrc[i] = (const char*)(Bbase + row * ld) + lchunk * 16;
  }
  const int steps = (int)(ld / 32);
  auto issue = [&](char* b, int s) {
    const int ko = s * ROWB;
#pragma unroll
    for (int i = 0; i < NIA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + ko), LDS_PTR(b + (wave * NIA + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NIB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[i] + ko), LDS_PTR(b + SA + (wave * NIB + i) * 1024), 16, 0,
                                       0);
  };
  // P V: each key tile's TPN scale loads are issued at the tile's first step, after its DMA
  // refill; a wait for step s's loads then allows 2 * NI newer loads, plus those TPN at the
  // three steps after a tile's first one
  auto sync_step = [&](int s, int u) {
    if (s + STAGES - 2 < steps) {
      if (PV && u != 0)
        wait_vm_lgkm0<2 * NI + TPN>();
      else
        wait_vm_lgkm0<2 * NI>();
    } else {
      wait_vm_lgkm0<0>();
    }
    __builtin_amdgcn_s_barrier();
  };

  f32x4_t acc[TCN][TPN];
#pragma unroll
  for (int ic = 0; ic < TCN; ++ic)
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) acc[ic][ip] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the queries of this lane's accumulator columns
  int qcol[TPN];
#pragma unroll
  for (int ip = 0; ip < TPN; ++ip) qcol[ip] = min(n0 + wn * TN + ip * 16 + (lane & 15), S - 1);
  float gcur[TPN], gnext[TPN];
  auto load_g = [&](float* g, int t) {
    const int tt = min(t, a.nkt - 1);
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) g[ip] = a.fac[((int64_t)fr * a.nkt + tt) * S + qcol[ip]];
  };
  if constexpr (PV) load_g(gcur, 0);
  const int rslot = ((lane >> 4) ^ (((lane & 15) >> 1) & 3)) * 16 + (lane & 15) * ROWB;
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < steps) issue(bufs[p], p);
  // STAGES = 4 steps of 32 keys = one 128-key tile per pass
  for (int sb = 0; sb < steps; sb += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int s = sb + u;
      if (s < steps) {
        sync_step(s, u);
        if (s + STAGES - 1 < steps) issue(bufs[(u + STAGES - 1) % STAGES], s + STAGES - 1);
        if (PV && u == 0) load_g(gnext, sb / STAGES + 1);
        const char* b = bufs[u];
        uint4 af[TCN], bf[TPN];
#pragma unroll
        for (int ic = 0; ic < TCN; ++ic) af[ic] = *(const uint4*)(b + (wm * TM + ic * 16) * ROWB + rslot);
#pragma unroll
        for (int ip = 0; ip < TPN; ++ip) bf[ip] = *(const uint4*)(b + SA + (wn * TN + ip * 16) * ROWB + rslot);
#pragma unroll
        for (int ip = 0; ip < TPN; ++ip)
#pragma unroll
          for (int ic = 0; ic < TCN; ++ic) Mma<T>::run(acc[ic][ip], af[ic], bf[ip]);
      }
    }
    if constexpr (PV) {
      // the 128-key tile of these four steps is in: scale by its g
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip) {
#pragma unroll
        for (int ic = 0; ic < TCN; ++ic)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[ic][ip][e] *= gcur[ip];
        gcur[ip] = gnext[ip];
      }
    }
  }
  wait_vm_lgkm0<0>();

  if constexpr (PV) {
    // O[i][c .. c + 3], rounded once
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) {
      const int i = n0 + wn * TN + ip * 16 + (lane & 15);
      if (i >= S) continue;
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) {
        const int c = m0 + wm * TM + ic * 16 + 4 * (lane >> 4);
        if (c < C) {
          uint2 pk;
          pk.x = pack2_bf16(acc[ic][ip][0], acc[ic][ip][1]);
          pk.y = pack2_bf16(acc[ic][ip][2], acc[ic][ip][3]);
          *(uint2*)((T*)a.o + ((int64_t)fr * S + i) * C + c) = pk;
        }
      }
    }
  } else {
    // softmax of each 128-key tile: scores in base 2, the keys past S masked. A tile is one
    // wave's rows (WPT = 1) or those of two waves, combined through LDS (WPT = 2).
    float* red = (float*)s0;  // [WGM][BN] per-wave maxima, then sums
    const int jb = m0 + wm * TM + 4 * (lane >> 4);
#pragma unroll
    for (int ic = 0; ic < TCN; ++ic)
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[ic][ip][e] = jb + ic * 16 + e < S ? acc[ic][ip][e] * a.sc : -INFINITY;
    float mx[TPN];
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) {
      float m = -INFINITY;
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, acc[ic][ip][e]);
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      mx[ip] = m;
    }
    if constexpr (WPT == 2) {
      __syncthreads();  // every wave is done with the stage buffers
      if ((lane >> 4) == 0) {
#pragma unroll
        for (int ip = 0; ip < TPN; ++ip) red[wm * BN + wn * TN + ip * 16 + lane] = mx[ip];
      }
      __syncthreads();
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip) {
        const int q = wn * TN + ip * 16 + (lane & 15), w0 = wm & ~1;
        mx[ip] = fmaxf(red[w0 * BN + q], red[(w0 + 1) * BN + q]);
      }
    }
    float sm[TPN];
#pragma unroll
    for (int ip = 0; ip < TPN; ++ip) {
      const int i = n0 + wn * TN + ip * 16 + (lane & 15);
      float l = 0.f;
#pragma unroll
      for (int ic = 0; ic < TCN; ++ic) {
        const float p0 = __builtin_amdgcn_exp2f(acc[ic][ip][0] - mx[ip]);
        const float p1 = __builtin_amdgcn_exp2f(acc[ic][ip][1] - mx[ip]);
        const float p2 = __builtin_amdgcn_exp2f(acc[ic][ip][2] - mx[ip]);
        const float p3 = __builtin_amdgcn_exp2f(acc[ic][ip][3] - mx[ip]);
        uint2 pk;
        pk.x = pack2_bf16(p0, p1);
        pk.y = pack2_bf16(p2, p3);
        l += __uint_as_float(pk.x << 16) + __uint_as_float(pk.x & 0xffff0000u) + __uint_as_float(pk.y << 16) +
             __uint_as_float(pk.y & 0xffff0000u);
        const int j = jb + ic * 16;  // 4 keys j .. j + 3: consecutive slots of V^T's order
        if (i < S && j < Sp) *(uint2*)((T*)a.p + ((int64_t)fr * S + i) * Sp + vt_slot(j)) = pk;
      }
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      sm[ip] = l;
    }
    if constexpr (WPT == 2) {
      __syncthreads();
      if ((lane >> 4) == 0) {
#pragma unroll
        for (int ip = 0; ip < TPN; ++ip) red[wm * BN + wn * TN + ip * 16 + lane] = sm[ip];
      }
      __syncthreads();
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip) {
        const int q = wn * TN + ip * 16 + (lane & 15), w0 = wm & ~1;
        sm[ip] = red[w0 * BN + q] + red[(w0 + 1) * BN + q];
      }
    }
    // (m_t, l_t) of this wave's 128-key tile (with WPT = 2, the even wave of the pair stores)
    const int t = (m0 + wm * TM) / KT;
    if ((WPT == 1 || (wm & 1) == 0) && (lane >> 4) == 0) {
#pragma unroll
      for (int ip = 0; ip < TPN; ++ip) {
        const int i = n0 + wn * TN + ip * 16 + lane;
        if (i < S && t < a.nkt) a.ml[((int64_t)fr * a.nkt + t) * S + i] = make_float2(mx[ip], sm[ip]);
      }
    }
  }
}

// Per query: M = max_t m_t, L = sum_t l_t 2^(m_t - M), f_t = max(2^(m_t - M) / L, 2^-100),
// stored as the P V kernel's scales g_t = f_t / f_t+1 and, for the last tile, f_t.
__global__ void __launch_bounds__(256) k_attn_fac(const AttnMatArgs a) {
  const int64_t n = (int64_t)a.nfr * a.S;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n) return;
  const int64_t fr = u / a.S, i = u - fr * a.S;
  const float2* ml = a.ml + fr * a.nkt * a.S + i;
  float M = -INFINITY;
  for (int t = 0; t < a.nkt; ++t) M = fmaxf(M, ml[(int64_t)t * a.S].x);
  float L = 0.f;
  for (int t = 0; t < a.nkt; ++t) L += ml[(int64_t)t * a.S].y * exp2f(ml[(int64_t)t * a.S].x - M);
  const float inv = 1.f / L, fmin_ = 0x1p-100f;
  float* g = a.fac + fr * a.nkt * a.S + i;
  float f = fmaxf(exp2f(ml[0].x - M) * inv, fmin_);
  for (int t = 0; t + 1 < a.nkt; ++t) {
    const float fn = fmaxf(exp2f(ml[(int64_t)(t + 1) * a.S].x - M) * inv, fmin_);
    g[(int64_t)t * a.S] = f / fn;
    f = fn;
  }
  g[(int64_t)(a.nkt - 1) * a.S] = f;
}

// ------------------------------------------------------------------ small kernels

template <typename S>
__device__ __forceinline__ float load_as_f32(const S* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<bf16_t>(const bf16_t* p, int64_t i) {
  return bf2f(p[i].u);
}

template <typename S, typename D>
__global__ void k_repack(const S* w, D* wp, int Cout, int Cin, int taps) {
  const int64_t n = (int64_t)Cout * Cin * taps;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int ci = (int)(idx % Cin);
    const int64_t r = idx / Cin;
    const int tap = (int)(r % taps);
    const int64_t o = r / taps;
    Elem<D>::st(wp + idx, load_as_f32<S>(w, (o * Cin + ci) * taps + tap));
  }
}

template <typename S>
__global__ void k_to_f32(const S* x, float* y, int64_t n, int bf) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float v = load_as_f32<S>(x, i);
    y[i] = bf ? bf2f(f2bf(v)) : v;
  }
}

template <typename S, typename D>
__global__ void k_ncthw_to_frames(const S* x, D* y, int B, int C, int Cp, int T, int H, int W) {
  const int64_t n = (int64_t)T * B * H * W * Cp;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(idx % Cp);
    int64_t r = idx / Cp;
    const int xx = (int)(r % W);
    r /= W;
    const int yy = (int)(r % H);
    r /= H;
    const int b = (int)(r % B);
    const int t = (int)(r / B);
    const float v = c < C ? load_as_f32<S>(x, ((((int64_t)b * C + c) * T + t) * H + yy) * W + xx) : 0.f;
    Elem<D>::st(y + idx, v);
  }
}

template <typename D>
__global__ void k_frames_to_ncthw(const D* x, D* y, int B, int C, int T, int H, int W) {
  const int64_t n = (int64_t)B * C * T * H * W;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int xx = (int)(idx % W);
    int64_t r = idx / W;
    const int yy = (int)(r % H);
    r /= H;
    const int t = (int)(r % T);
    r /= T;
    const int c = (int)(r % C);
    const int b = (int)(r / C);
    y[idx] = x[((((int64_t)t * B + b) * H + yy) * W + xx) * C + c];
  }
}

// ------------------------------------------------------------------ launchers

static int grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  return (int)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

template <typename T, int TC, int TP>
static hipError_t conv_go(const ConvArgs& a, hipStream_t s) {
  const int64_t M = (int64_t)a.F * a.B * a.Ho * a.Wo;
  const int64_t blocks = ((a.Cout + TC - 1) / TC) * ((M + TP - 1) / TP);
  hipLaunchKernelGGL((k_conv<T, TC, TP>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int TC, int TP, int WGC, int WGP, int STAGES, int MINB, bool RB2 = false, typename T = bf16_t>
static hipError_t conv_dma_launch(const ConvArgs& a, hipStream_t s) {
  const int64_t M = (int64_t)a.F * a.B * a.Ho * a.Wo;
  const int64_t blocks = ((a.Cout + TC - 1) / TC) * ((M + TP - 1) / TP) * a.ksplit;
  constexpr int KS = 64 / (int)sizeof(T);  // channels per K step
  // the aligned path loads every wave's weight rows unconditionally: only where they all lie
  // in the tile (16 rows per wave and instruction), not on the 16-channel tile
  if constexpr (TC >= 16 * WGC * WGP) {
    if (a.Cin % KS == 0 && a.Cout % TC == 0) {
      hipLaunchKernelGGL((k_conv_dma<TC, TP, WGC, WGP, STAGES, MINB, true, RB2, T>), dim3((unsigned)blocks),
                         dim3(64 * WGC * WGP), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_conv_dma<TC, TP, WGC, WGP, STAGES, MINB, false, RB2, T>), dim3((unsigned)blocks),
                     dim3(64 * WGC * WGP), 0, s, a);
  return hipGetLastError();
}

template <int TC, int TP, int WGC, int WGP, int STAGES, int MINB, bool RB2 = false, typename T = bf16_t>
static hipError_t conv_dma_go(const ConvArgs& a, hipStream_t s) {
  if (hipError_t e = conv_dma_launch<TC, TP, WGC, WGP, STAGES, MINB, RB2, T>(a, s)) return e;
  if (a.ksplit > 1) {
    const int64_t units = (int64_t)a.F * a.B * a.Ho * a.Wo * (a.Cout / 8);
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int TC, int TPY, int TPX, int WGC, int WGP>
static hipError_t conv_halo_go(const ConvArgs& a, hipStream_t s) {
  const int64_t blocks =
      (int64_t)((a.Cout + TC - 1) / TC) * ((a.Wo + TPX - 1) / TPX) * ((a.Ho + TPY - 1) / TPY) * a.F * a.B * a.ksplit;
  if (a.up)
    hipLaunchKernelGGL((k_conv_halo<TC, TPY, TPX, WGC, WGP, true>), dim3((unsigned)blocks), dim3(64 * WGC * WGP), 0, s, a);
  else
    hipLaunchKernelGGL((k_conv_halo<TC, TPY, TPX, WGC, WGP, false>), dim3((unsigned)blocks), dim3(64 * WGC * WGP), 0, s, a);
  if (hipError_t e = hipGetLastError()) return e;
  if (a.ksplit > 1) {
    const int64_t units = (int64_t)a.F * a.B * a.Ho * a.Wo * (a.Cout / 8);
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

bool conv_halo_supported(const ConvArgs& a, int dtype, int tile) {
  // the kernel addresses an input frame with 32-bit byte offsets and marks padding with the
  // offset 2^31: a frame (one batch element) must hold fewer bytes than that
  const bool small = (int64_t)a.Hin * a.Win * a.Cin * 2 < ((int64_t)1 << 31);
  const bool geometry = dtype == kBF16 && small && a.kh == 3 && a.kw == 3 && (a.kt == 1 || a.kt == 3) &&
                        a.Cin % 32 == 0 &&
                        (!a.up || (a.Ho % 2 == 0 && a.Wo % 2 == 0 && a.Hin * 2 == a.Ho && a.Win * 2 == a.Wo)) &&
                        (a.up || (a.Hin == a.Ho && a.Win == a.Wo));
  if (tile == kTileHalo16x16x32)  // conv_out: up to 16 channels, the unpatchify + clamp store
    return geometry && a.Cout <= 16 && a.Cout % 4 == 0 && a.mode == kEpiVideo;
  return geometry && a.Cout % 128 == 0 && (a.mode == kEpiFrames || a.mode == kEpiFramesF32);
}

hipError_t launch_conv(const ConvArgs& a, int dtype, int tile, hipStream_t s) {
  if (tile == kTileHalo128x16x32) {
    if (!conv_halo_supported(a, dtype, tile)) return hipErrorInvalidValue;
    return conv_halo_go<128, 16, 32, 2, 4>(a, s);
  }
  if (tile == kTileHalo16x16x32) {
    if (!conv_halo_supported(a, dtype, tile)) return hipErrorInvalidValue;
    return conv_halo_go<16, 16, 32, 1, 8>(a, s);
  }
  if (tile == kTileHalo128x32x16) {
    if (!conv_halo_supported(a, dtype, tile)) return hipErrorInvalidValue;
    return conv_halo_go<128, 32, 16, 2, 4>(a, s);
  }
  if (tile == kTileHalo128x16x16) {
    if (!conv_halo_supported(a, dtype, tile)) return hipErrorInvalidValue;
    return conv_halo_go<128, 16, 16, 2, 4>(a, s);
  }
  if (dtype == kBF16) {
    if (tile == kTileDma256x128) return conv_dma_go<256, 128, 2, 2, 3, 2>(a, s);
    if (tile == kTileDma256x256) return conv_dma_go<256, 256, 2, 2, 4, 1, true>(a, s);
    if (tile == kTileDma128x256) return conv_dma_go<128, 256, 2, 2, 3, 2>(a, s);
    if (tile == kTileDma128x128) return conv_dma_go<128, 128, 2, 2, 4, 2>(a, s);
    if (tile == kTileDma16x256) return conv_dma_go<16, 256, 1, 4, 4, 2>(a, s);
    if (tile == kTileDma256x256w8) return conv_dma_go<256, 256, 2, 4, 4, 1>(a, s);
    if (tile == kTileDma256x256w8b) return conv_dma_go<256, 256, 4, 2, 4, 1>(a, s);
    if (tile == kTile32x256) return conv_go<bf16_t, 32, 256>(a, s);
    if (tile == kTile256x128) return conv_go<bf16_t, 256, 128>(a, s);
    return conv_go<bf16_t, 128, 128>(a, s);
  }
  // fp32 on the direct-to-LDS tiles (16 channels per K step; no split K, no staging epilogue)
  if (tile == kTileDma256x128) return conv_dma_go<256, 128, 2, 2, 3, 2, false, float>(a, s);
  if (tile == kTileDma256x256) return conv_dma_go<256, 256, 2, 2, 4, 1, true, float>(a, s);
  if (tile == kTileDma128x256) return conv_dma_go<128, 256, 2, 2, 3, 2, false, float>(a, s);
  if (tile == kTileDma128x128) return conv_dma_go<128, 128, 2, 2, 4, 2, false, float>(a, s);
  if (tile == kTileDma16x256) return conv_dma_go<16, 256, 1, 4, 4, 2, false, float>(a, s);
  if (tile == kTileDma256x256w8) return conv_dma_go<256, 256, 2, 4, 4, 1, false, float>(a, s);
  if (tile == kTileDma256x256w8b) return conv_dma_go<256, 256, 4, 2, 4, 1, false, float>(a, s);
  if (tile == kTile32x256) return conv_go<float, 32, 256>(a, s);
  return conv_go<float, 128, 128>(a, s);
}

template <typename T, int LPP, int VPL>
static hipError_t norm_v_go(const NormArgs& a, hipStream_t s) {
  constexpr int R = 4;
  if constexpr (sizeof(T) == 2) {
    // bf16 with SiLU over at least two rounds of 16-wave blocks (or where asked for): the
    // table variant, two workgroups per CU
    constexpr int TPB = 16 * (64 / LPP) * R;
    const int64_t nall = (int64_t)((a.HW + TPB - 1) / TPB) * a.F * a.B;
    if (a.silu && (a.tab > 0 || (a.tab < 0 && nall >= 1024))) {
      hipLaunchKernelGGL((k_norm_v<T, LPP, VPL, R, true, true, 16>), dim3(512), dim3(1024), 0, s, a);
      return hipGetLastError();
    }
  }
  const int per_block = 4 * (64 / LPP) * R;
  const dim3 grid((unsigned)((a.HW + per_block - 1) / per_block), (unsigned)(a.F * a.B));
  if (a.silu)
    hipLaunchKernelGGL((k_norm_v<T, LPP, VPL, R, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_norm_v<T, LPP, VPL, R, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm(const NormArgs& a, int dtype, hipStream_t s) {
  if (dtype == kBF16) {
    switch (a.C) {
      case 16: return norm_v_go<bf16_t, 2, 1>(a, s);
      case 32: return norm_v_go<bf16_t, 4, 1>(a, s);
      case 64: return norm_v_go<bf16_t, 8, 1>(a, s);
      case 128: return norm_v_go<bf16_t, 16, 1>(a, s);
      case 256: return norm_v_go<bf16_t, 32, 1>(a, s);
      case 512: return norm_v_go<bf16_t, 32, 2>(a, s);
      case 1024: return norm_v_go<bf16_t, 64, 2>(a, s);
    }
  } else {
    switch (a.C) {
      case 16: return norm_v_go<float, 4, 1>(a, s);
      case 32: return norm_v_go<float, 8, 1>(a, s);
      case 64: return norm_v_go<float, 16, 1>(a, s);
      case 128: return norm_v_go<float, 32, 1>(a, s);
      case 256: return norm_v_go<float, 64, 1>(a, s);
      case 512: return norm_v_go<float, 64, 2>(a, s);
      case 1024: return norm_v_go<float, 64, 4>(a, s);
    }
  }
  const int64_t M = (int64_t)a.F * a.B * a.HW;
  const unsigned blocks = (unsigned)((M + 3) / 4);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_norm<bf16_t>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_norm<float>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int NW, int DW>
static hipError_t attn_go(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_attn<T, NW, DW>), dim3((unsigned)((a.S + 31) / 32), (unsigned)a.nfr, (unsigned)a.ksplit),
                     dim3(64 * NW), 0, s, a);
  if (a.ksplit > 1) {
    if (hipError_t e = hipGetLastError()) return e;
    const int64_t units = (int64_t)a.nfr * a.S * (a.C / 4);
    hipLaunchKernelGGL((k_attn_combine<T>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool attn_supported(int C, int dtype) {
  (void)dtype;
  return C == 64 || C == 128 || C == 256 || C == 384 || C == 512 || C == 1024;
}

hipError_t launch_attn(const AttnArgs& a, int dtype, hipStream_t s) {
  if (dtype == kBF16) {
    switch (a.C) {
      case 64: return attn_go<bf16_t, 2, 32>(a, s);
      case 128: return attn_go<bf16_t, 4, 32>(a, s);
      case 256: return attn_go<bf16_t, 4, 64>(a, s);
      case 384: return attn_go<bf16_t, 4, 96>(a, s);
      case 512: return attn_go<bf16_t, 4, 128>(a, s);
      case 1024: return attn_go<bf16_t, 8, 128>(a, s);
    }
  } else {
    switch (a.C) {
      case 64: return attn_go<float, 4, 16>(a, s);
      case 128: return attn_go<float, 8, 16>(a, s);
      case 256: return attn_go<float, 8, 32>(a, s);
      case 384: return attn_go<float, 8, 48>(a, s);
      case 512: return attn_go<float, 8, 64>(a, s);
      case 1024: return attn_go<float, 8, 128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

// A tile shape's workgroups for one of the two GEMMs: the 256 x 256 tiles where they give
// the chip at least two rounds of workgroups (one per CU), else 128 x 128 (two per CU).
hipError_t launch_attn_mm(const AttnMatArgs& a, hipStream_t s) {
  if (a.C % 64 != 0 || a.Sp % 32 != 0 || a.Sp < a.S || a.nkt != (a.S + 127) / 128) return hipErrorInvalidValue;
  auto blocks = [&](int64_t rows, int tile) { return (int64_t)a.nfr * ((rows + tile - 1) / tile) * ((a.S + tile - 1) / tile); };
  const int64_t s256 = blocks(a.S, 256), p256 = blocks(a.C, 256);
  if (blocks(a.S, 128) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (s256 >= 512)
    hipLaunchKernelGGL((k_attn_mm<0, 256, 256, 2, 4>), dim3((unsigned)s256), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_mm<0, 128, 128, 2, 2>), dim3((unsigned)blocks(a.S, 128)), dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError()) return e;
  const int64_t n = (int64_t)a.nfr * a.S;
  hipLaunchKernelGGL(k_attn_fac, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError()) return e;
  if (p256 >= 512)
    hipLaunchKernelGGL((k_attn_mm<1, 256, 256, 2, 4>), dim3((unsigned)p256), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_mm<1, 128, 128, 2, 2>), dim3((unsigned)blocks(a.C, 128)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_repack(const void* w, int src_dtype, void* dst, int dst_dtype, int Cout, int Cin, int taps,
                         hipStream_t s) {
  const int g = grid_for((int64_t)Cout * Cin * taps, 256);
  if (src_dtype == kF32 && dst_dtype == kF32)
    hipLaunchKernelGGL((k_repack<float, float>), dim3(g), dim3(256), 0, s, (const float*)w, (float*)dst, Cout, Cin, taps);
  else if (src_dtype == kF32)
    hipLaunchKernelGGL((k_repack<float, bf16_t>), dim3(g), dim3(256), 0, s, (const float*)w, (bf16_t*)dst, Cout, Cin, taps);
  else if (dst_dtype == kF32)
    hipLaunchKernelGGL((k_repack<bf16_t, float>), dim3(g), dim3(256), 0, s, (const bf16_t*)w, (float*)dst, Cout, Cin, taps);
  else
    hipLaunchKernelGGL((k_repack<bf16_t, bf16_t>), dim3(g), dim3(256), 0, s, (const bf16_t*)w, (bf16_t*)dst, Cout, Cin, taps);
  return hipGetLastError();
}

hipError_t launch_to_f32(const void* x, int src_dtype, float* dst, int64_t n, int dtype, hipStream_t s) {
  const int g = grid_for(n, 256);
  if (src_dtype == kF32)
    hipLaunchKernelGGL(k_to_f32<float>, dim3(g), dim3(256), 0, s, (const float*)x, dst, n, dtype == kBF16 ? 1 : 0);
  else
    hipLaunchKernelGGL(k_to_f32<bf16_t>, dim3(g), dim3(256), 0, s, (const bf16_t*)x, dst, n, dtype == kBF16 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_ncthw_to_frames(const void* x, int src_dtype, void* dst, int dst_dtype, int B, int C, int Cp, int T,
                                  int H, int W, hipStream_t s) {
  const int g = grid_for((int64_t)T * B * H * W * Cp, 256);
  if (src_dtype == kF32 && dst_dtype == kF32)
    hipLaunchKernelGGL((k_ncthw_to_frames<float, float>), dim3(g), dim3(256), 0, s, (const float*)x, (float*)dst, B, C, Cp, T, H, W);
  else if (src_dtype == kF32)
    hipLaunchKernelGGL((k_ncthw_to_frames<float, bf16_t>), dim3(g), dim3(256), 0, s, (const float*)x, (bf16_t*)dst, B, C, Cp, T, H, W);
  else if (dst_dtype == kF32)
    hipLaunchKernelGGL((k_ncthw_to_frames<bf16_t, float>), dim3(g), dim3(256), 0, s, (const bf16_t*)x, (float*)dst, B, C, Cp, T, H, W);
  else
    hipLaunchKernelGGL((k_ncthw_to_frames<bf16_t, bf16_t>), dim3(g), dim3(256), 0, s, (const bf16_t*)x, (bf16_t*)dst, B, C, Cp, T, H, W);
  return hipGetLastError();
}

hipError_t launch_frames_to_ncthw(const void* x, void* dst, int dtype, int B, int C, int T, int H, int W,
                                  hipStream_t s) {
  const int g = grid_for((int64_t)B * C * T * H * W, 256);
  if (dtype == kF32)
    hipLaunchKernelGGL(k_frames_to_ncthw<float>, dim3(g), dim3(256), 0, s, (const float*)x, (float*)dst, B, C, T, H, W);
  else
    hipLaunchKernelGGL(k_frames_to_ncthw<bf16_t>, dim3(g), dim3(256), 0, s, (const bf16_t*)x, (bf16_t*)dst, B, C, T, H, W);
  return hipGetLastError();
}

}  // namespace wanvae
