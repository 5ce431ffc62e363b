// Internal interface between the host orchestrator (wanvae.cpp) and the gfx950 kernels
// (kernels.hip). Activations live in HBM as channels-last frames: one frame of a
// level is [B][H][W][C] contiguous, and a kernel addresses frame s through a table of
// frame pointers (nullptr = a zero frame). The causal caches are therefore read in
// place: a conv's table lists its history frames, then the chunk's frames, wherever
// they live.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "wanvae.h"

namespace wanvae {

constexpr int kMaxFrames = 8;  // 2 history frames + up to 4 chunk frames, or 8 interleaved outputs

enum Dtype { kF32 = 0, kBF16 = 1 };

// Epilogue of the conv kernel: where and how the accumulated result is written.
enum Epilogue {
  kEpiFrames = 0,      // out frame t, channel c
  kEpiInterleave = 1,  // time conv: channel c < outC -> frame 2t, channel outC + c -> frame 2t+1
  kEpiVideo = 2,       // unpatchify + clamp into the NCTHW video
  kEpiQKV = 3,         // 1x1 conv C -> 3C: q, k as [frame][S][C], v transposed as [frame][C][Sp]
  kEpiFramesF32 = 4,   // as kEpiFrames, but the float32 sums + bias are stored unrounded as float32
                       // (a bf16 conv with a float32 output; no residual or DupUp3D term)
};

struct ConvArgs {
  // input frames of the time-padded sequence (history zeros as nullptr), batch strides in elements
  const void* in[kMaxFrames];
  int64_t in_bs[kMaxFrames];
  int B, Hin, Win, Cin;   // input frame geometry
  int Ho, Wo, Cout;       // output geometry
  int kt, kh, kw;         // kernel (kt in {1,3}; kh, kw in {1,3})
  int up;                 // 1: the input is read through nearest x2 upsampling (Hin = Ho/2)
  int F;                  // output frames
  const void* w;          // [Cout][kt][kh][kw][Cin], compute type
  const float* bias;      // [Cout], value already rounded to the compute type
  int mode;               // Epilogue
  void* out[kMaxFrames];
  int64_t out_bs[kMaxFrames];
  int outC;               // channels of an output frame (Cout, Cout/2 interleaved, C for QKV)
  int has_res;            // += residual frame (same layout as out), each sum rounded
  const void* res[kMaxFrames];
  int64_t res_bs[kMaxFrames];
  int has_dup;            // += DupUp3D of the block input at (Ho/2, Wo/2)
  const void* dup[kMaxFrames];
  int64_t dup_bs[kMaxFrames];
  int dup_C, dup_r, dup_ft, dup_shift;
  void* video;            // kEpiVideo: [B][3][vF][2Ho][2Wo]
  int vF, vf0;
  void* q;                // kEpiQKV
  void* k;
  void* vt;
  int S, Sp;
  int ksplit;             // >= 1: K ranges of the direct-to-LDS kernels (> 1: bf16, Cout % 8 == 0,
  float* part;            //   not the video epilogue); float32 partials [ksplit][M][Cout]
};

struct NormArgs {
  const void* in[kMaxFrames];
  int64_t in_bs[kMaxFrames];
  void* out[kMaxFrames];
  int64_t out_bs[kMaxFrames];
  int F, B, HW, C;
  const float* gamma;  // [C], rounded to the compute type
  float sqrtC;         // sqrt(C) as a float
  int silu;
  int tab;             // bf16 SiLU from the LDS table: -1 where the launch is large, 0 never, 1 always
};

struct AttnArgs {
  const void* q;   // [nfr][S][C]
  const void* k;   // [nfr][S][C]
  const void* vt;  // [nfr][C][Sp], zero beyond S
  void* o;         // [nfr][S][C]
  int nfr, S, Sp, C;
  float scale;     // 1/sqrt(C)
  int ksplit;      // key ranges (> 1: the partial results go to opart / ml, then a combine pass)
  float* opart;    // [ksplit][nfr][S][C] unnormalised O of each key range
  float* ml;       // [ksplit][nfr][S][2] running max (base-2 units) and sum of each key range
};

// The bf16 attention core with the scores materialised (kernels.hip, k_attn_mm): q, k, vt as
// for AttnArgs; p [nfr][S][Sp] bf16 (the tile-relative softmax numerators, keys in V^T's slot
// order), ml [nfr][nkt][S] (each 128-key tile's max and sum per query), fac [nfr][nkt][S] (each
// tile's weight per query), o [nfr][S][C]. nkt = ceil(S / 128).
struct AttnMatArgs {
  const void* q;
  const void* k;
  const void* vt;
  void* p;
  float2* ml;
  float* fac;
  void* o;
  int nfr, S, Sp, C, nkt;
  float sc;  // 1/sqrt(C) * log2(e)
};

// Tile shapes of the conv kernel: channels x positions per workgroup.
enum ConvTile {
  kTile128x128 = 0,  // register-staged loads (bf16 and fp32)
  kTile32x256 = 1,   // small Cout (conv_out, post_quant_conv)
  kTile256x128 = 2,
  kTileDma256x128 = 3,  // bf16, direct-to-LDS pipeline
  kTileDma256x256 = 4,
  kTileDma128x128 = 5,
  kTileDma128x256 = 6,
  kTileDma16x256 = 7,   // bf16, small Cout (conv_out)
  kTileDma256x256w8 = 8,   // 8 waves, 128 x 64 per wave
  kTileDma256x256w8b = 9,  // 8 waves, 64 x 128 per wave
  kTileHalo128x16x32 = 10, // bf16 3x3 convs: 128 channels x a 16 x 32 block, input patch reused over the taps
  kTileHalo16x16x32 = 11,  // the same for conv_out (up to 16 channels, the video store)
  kTileHalo128x16x16 = 12, // 128 channels x a 16 x 16 block (small frames, with split K)
  kTileHalo128x32x16 = 13, // 128 channels x a 32 x 16 block (frames that 16-column blocks pad less)
};

// One tile of the tiled decode (tiles.hip): the decoded tile cur [planes][H][W] (planes = batch x
// colour x frame) takes the ramp with the composed tile above (its last Ev of Ha rows) over its
// first Ev rows, then with the composed tile to the left (its last Eh of Wl columns) over its
// first Eh columns, in place; its rows [0, keep_h) x columns [0, keep_w) go to the video
// [planes][VH][VW] at (oy, ox). above / left may be nullptr (no ramp).
struct TileBlendArgs {
  void* cur;
  const void* above;
  const void* left;
  int64_t planes;
  int H, W, Ha, Ev, Wl, Eh;
  void* video;
  int VH, VW, oy, ox, keep_h, keep_w;
};
hipError_t launch_tile_blend(const TileBlendArgs& a, int dtype, hipStream_t s);
// rows x row_bytes bytes: dst + r * dst_pitch <- src + r * src_pitch (pitches in bytes); the
// regions must not overlap
hipError_t launch_copy_rows(const void* src, int64_t src_pitch, void* dst, int64_t dst_pitch, int64_t row_bytes,
                            int64_t rows, hipStream_t s);
// src [planes][h][w] (elements of esize bytes) rows y0.. x columns x0.. -> dst [planes][th][tw]
hipError_t launch_crop(const void* src, void* dst, int esize, int64_t planes, int h, int w, int y0, int x0, int th,
                       int tw, hipStream_t s);

hipError_t launch_conv(const ConvArgs& a, int dtype, int tile, hipStream_t s);
// whether a halo-tile kernel handles this conv (bf16, 3x3 spatial, Cin % 32, an input frame of
// fewer than 2^31 bytes; tiles 10, 12, 13: Cout % 128 and a frame epilogue; tile 11: Cout <= 16
// and the video epilogue)
bool conv_halo_supported(const ConvArgs& a, int dtype, int tile);
hipError_t launch_norm(const NormArgs& a, int dtype, hipStream_t s);
bool attn_supported(int C, int dtype);
// bf16 only; C % 64 == 0, Sp a multiple of 32 >= S
hipError_t launch_attn_mm(const AttnMatArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int dtype, hipStream_t s);
// w [Cout][Cin][taps] (src dtype) -> [Cout][taps][Cin] (dst dtype), rounded to nearest even
hipError_t launch_repack(const void* w, int src_dtype, void* dst, int dst_dtype, int Cout, int Cin, int taps,
                         hipStream_t s);
// n values (src dtype) -> float, rounded to the compute dtype first
hipError_t launch_to_f32(const void* x, int src_dtype, float* dst, int64_t n, int dtype, hipStream_t s);
// NCTHW [B][C][T][H][W] (src dtype) -> frames [T][B][H][W][Cp] (dst dtype), channels >= C zero
hipError_t launch_ncthw_to_frames(const void* x, int src_dtype, void* dst, int dst_dtype, int B, int C, int Cp, int T,
                                  int H, int W, hipStream_t s);
// frames [T][B][H][W][C] -> NCTHW [B][C][T][H][W], same dtype
hipError_t launch_frames_to_ncthw(const void* x, void* dst, int dtype, int B, int C, int T, int H, int W,
                                  hipStream_t s);

// The single causal conv in two halves (wanvae.cpp), for entry points that bring their own
// device memory: conv_plan validates the arguments of wanvae_causal_conv3d and reports the
// workspace the conv needs; conv_enqueue enqueues it on `ws` (at least that many bytes).
int conv_plan(const void* x, const void* cache, int64_t B, int64_t Cin, int64_t t, int64_t h, int64_t w,
              int64_t n_cache, const wanvae_tensor* weight, const wanvae_tensor* bias, int32_t layout, int32_t dtype,
              const void* y, int32_t y_dtype, const void* cache_out, size_t* need);
int conv_enqueue(const void* x, const void* cache, int64_t B, int64_t Cin, int64_t t, int64_t h, int64_t w,
                 int64_t n_cache, const wanvae_tensor* weight, const wanvae_tensor* bias, int32_t layout,
                 int32_t dtype, void* y, int32_t y_dtype, void* cache_out, void* ws, hipStream_t st);
// sets the calling thread's wanvae_last_error() message; returns code
int report(int code, const char* msg);

}  // namespace wanvae
