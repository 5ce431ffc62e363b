// Spatially tiled decode: the latent crop of a tile and the blend of the decoded tiles where
// they overlap (the diffusers PR page "Implement tiled VAE encoding/decoding for Wan model";
// the blend rule is not on the page and is read as a linear ramp with the composed tile above,
// then the composed tile to the left). Both are HBM-bound copies with a few flops per element.
// Also the strided row copy that writes a single causal conv's updated cache (the last two
// frames of cache ++ chunk, FastVideo's "wan22_vae_decode reference.py" page, "Causal caches").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "internal.h"

namespace wanvae {

namespace {

__device__ inline float ld_elem(const float* p, int64_t i) { return p[i]; }
__device__ inline float ld_elem(const uint16_t* p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

// float -> storage type, round to nearest even (bf16: on the bit pattern; NaN stays a quiet NaN)
__device__ inline float round_to(float v, const float*) { return v; }
__device__ inline float round_to(float v, const uint16_t*) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return __uint_as_float((u | 0x00400000u) & 0xffff0000u);
  return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}
__device__ inline void st_elem(float* p, int64_t i, float v) { p[i] = v; }
__device__ inline void st_elem(uint16_t* p, int64_t i, float v) { p[i] = (uint16_t)(__float_as_uint(v) >> 16); }

// One ramp step: other * (1 - y/E) + own * (y/E), weights as float32 constants computed in
// double (y/E, 1 - y/E), each product and the sum rounded to the storage type. The products
// and the sum are separate IEEE operations (no fused multiply-add).
template <typename T>
__device__ inline float ramp(float other, float own, int y, int E) {
  const double q = (double)y / (double)E;
  const float wo = (float)(1.0 - q), wn = (float)q;
  const T* tag = nullptr;
  return round_to(__fadd_rn(round_to(__fmul_rn(other, wo), tag), round_to(__fmul_rn(own, wn), tag)), tag);
}

template <typename T>
__global__ void __launch_bounds__(256) k_tile_blend(const TileBlendArgs a) {
  T* cur = (T*)a.cur;
  const T* above = (const T*)a.above;
  const T* left = (const T*)a.left;
  T* video = (T*)a.video;
  const int64_t n = (int64_t)a.planes * a.H * a.W;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int x = (int)(i % a.W);
    const int64_t r = i / a.W;
    const int y = (int)(r % a.H);
    const int64_t pl = r / a.H;  // (batch, colour, frame) plane
    float v = ld_elem(cur, i);
    bool changed = false;
    if (above && y < a.Ev) {
      v = ramp<T>(ld_elem(above, (pl * a.Ha + (a.Ha - a.Ev + y)) * a.W + x), v, y, a.Ev);
      changed = true;
    }
    if (left && x < a.Eh) {
      v = ramp<T>(ld_elem(left, (pl * a.H + y) * a.Wl + (a.Wl - a.Eh + x)), v, x, a.Eh);
      changed = true;
    }
    if (changed) st_elem(cur, i, v);
    if (y < a.keep_h && x < a.keep_w) st_elem(video, (pl * a.VH + a.oy + y) * a.VW + a.ox + x, v);
  }
}

// src [planes][h][w] (element type T) at rows y0.., columns x0.. -> dst [planes][th][tw]
template <typename T>
__global__ void __launch_bounds__(256) k_crop(const T* __restrict__ src, T* __restrict__ dst, int64_t planes, int h,
                                              int w, int y0, int x0, int th, int tw) {
  const int64_t n = planes * th * tw;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int x = (int)(i % tw);
    const int64_t r = i / tw;
    const int y = (int)(r % th);
    const int64_t p = r / th;
    dst[i] = src[(p * h + y0 + y) * w + x0 + x];
  }
}

// rows of units_per_row U-sized units: dst row r at dst + r * dp, src row r at src + r * sp
template <typename U>
__global__ void __launch_bounds__(256) k_copy_rows(const char* __restrict__ src, int64_t sp, char* __restrict__ dst,
                                                   int64_t dp, int64_t units_per_row, int64_t rows) {
  const int64_t n = units_per_row * rows;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / units_per_row, u = i - r * units_per_row;
    ((U*)(dst + r * dp))[u] = ((const U*)(src + r * sp))[u];
  }
}

int grid_for(int64_t n) { return (int)std::min<int64_t>((n + 255) / 256, 4096); }

}  // namespace

hipError_t launch_tile_blend(const TileBlendArgs& a, int dtype, hipStream_t s) {
  const int64_t n = (int64_t)a.planes * a.H * a.W;
  if (n <= 0) return hipSuccess;
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_tile_blend<uint16_t>, dim3(grid_for(n)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_tile_blend<float>, dim3(grid_for(n)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, int64_t src_pitch, void* dst, int64_t dst_pitch, int64_t row_bytes,
                            int64_t rows, hipStream_t s) {
  if (row_bytes <= 0 || rows <= 0) return hipSuccess;
  const uint64_t all = (uint64_t)(uintptr_t)src | (uint64_t)(uintptr_t)dst | (uint64_t)src_pitch |
                       (uint64_t)dst_pitch | (uint64_t)row_bytes;
  const char* sp = (const char*)src;
  char* dp = (char*)dst;
  if (all % 16 == 0) {
    const int64_t u = row_bytes / 16;
    hipLaunchKernelGGL(k_copy_rows<uint4>, dim3(grid_for(u * rows)), dim3(256), 0, s, sp, src_pitch, dp, dst_pitch, u,
                       rows);
  } else if (all % 4 == 0) {
    const int64_t u = row_bytes / 4;
    hipLaunchKernelGGL(k_copy_rows<uint32_t>, dim3(grid_for(u * rows)), dim3(256), 0, s, sp, src_pitch, dp,
                       dst_pitch, u, rows);
  } else {
    if (all % 2 != 0) return hipErrorInvalidValue;
    const int64_t u = row_bytes / 2;
    hipLaunchKernelGGL(k_copy_rows<uint16_t>, dim3(grid_for(u * rows)), dim3(256), 0, s, sp, src_pitch, dp,
                       dst_pitch, u, rows);
  }
  return hipGetLastError();
}

hipError_t launch_crop(const void* src, void* dst, int esize, int64_t planes, int h, int w, int y0, int x0, int th,
                       int tw, hipStream_t s) {
  const int64_t n = planes * th * tw;
  if (n <= 0) return hipSuccess;
  if (esize == 2)
    hipLaunchKernelGGL(k_crop<uint16_t>, dim3(grid_for(n)), dim3(256), 0, s, (const uint16_t*)src, (uint16_t*)dst,
                       planes, h, w, y0, x0, th, tw);
  else
    hipLaunchKernelGGL(k_crop<uint32_t>, dim3(grid_for(n)), dim3(256), 0, s, (const uint32_t*)src, (uint32_t*)dst,
                       planes, h, w, y0, x0, th, tw);
  return hipGetLastError();
}

}  // namespace wanvae
