/*
 * wanvae.h -- C ABI of the MI355X (gfx950) Wan2.2 TI2V-5B VAE decoder.
 *
 * The operation is the decoder of FastVideo's "wan22_vae_decode reference.py" page
 * (a standalone reference of diffusers' AutoencoderKLWan._decode): latents
 * z [B, 48, T, h, w] -> video [B, 3, 4T-3, 16h, 16w] in [-1, 1], decoded one latent
 * frame at a time with the causal caches (sections "What is computed", "The parts",
 * "The first latent frame yields one frame", "Causal caches", "Precision").
 *
 * Conventions shared by every entry point
 *  - All data pointers (z, video, x, cache, y, weight data, workspace) are DEVICE
 *    pointers on the current HIP device, owned by the caller. The library never frees
 *    them and keeps no reference after the call returns.
 *  - Calls are stream-ordered and asynchronous: `stream` is a hipStream_t (NULL = the
 *    null stream). A status of WANVAE_OK means every launch was enqueued; results are
 *    ready once the stream is synchronised.
 *  - dtype is the compute type: WANVAE_F32 (fp32 everywhere) or WANVAE_BF16 (bf16
 *    operands and storage, fp32 accumulation, at the rounding points the page's
 *    "Precision" section lists). Any other value -> WANVAE_EDTYPE (the page's ValueError).
 *    Weights of either dtype are accepted and rounded (nearest even) to the compute type.
 *  - Arguments are validated before anything is launched: on an error nothing has been
 *    enqueued. After an error the output contents are undefined.
 *  - Status codes are 0 or negative; wanvae_last_error() returns a message for the last
 *    failed call on the calling thread.
 *  - Workspace: `workspace` may be NULL, in which case the library allocates what it
 *    needs stream-ordered on `stream` (hipMallocAsync / hipFreeAsync). Otherwise it must
 *    hold at least the size the matching *_workspace_size function reports; smaller ->
 *    WANVAE_EWORKSPACE. One workspace must not be used by two calls that overlap in time.
 */
#ifndef WANVAE_H
#define WANVAE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types (wanvae_tensor.dtype, z_dtype and the compute dtype). */
#define WANVAE_F32 0
#define WANVAE_BF16 1

/* Activation layouts for the single-op entry points. */
#define WANVAE_NCTHW 0 /* [B, C, T, H, W], as on the page */
#define WANVAE_NTHWC 1 /* [B, T, H, W, C], channels last */

/* Status codes. */
#define WANVAE_OK 0
#define WANVAE_EDTYPE -1    /* dtype not WANVAE_F32 / WANVAE_BF16 */
#define WANVAE_EMISSING -2  /* a parameter the decoder needs is not in the table */
#define WANVAE_ESHAPE -3    /* a size or a parameter shape does not fit */
#define WANVAE_ETOPOLOGY -4 /* the parameter table is not a Wan2.2 decoder */
#define WANVAE_EWORKSPACE -5 /* workspace smaller than required */
#define WANVAE_EHIP -6      /* a HIP call failed (possibly an earlier asynchronous fault) */
#define WANVAE_EARG -7      /* NULL pointer, duplicate name or other invalid argument */

/* One parameter: diffusers' name, a device pointer to contiguous data, its element type
 * and shape (ndim <= 5). */
typedef struct {
  const char *name;
  const void *data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[5];
} wanvae_tensor;

/*
 * wanvae_decode -- the whole decoder (the page's decode(z, weights, dtype)).
 *
 *  z        [B, 48, T, h, w] NCTHW, element type z_dtype (rounded to dtype first).
 *  weights  n_weights parameters. Names beginning with "decoder." or "post_quant_conv."
 *           are used; all others are ignored. The 110 tensors of the decoder must be
 *           present (else WANVAE_EMISSING) with the shapes of diffusers' state dict
 *           (else WANVAE_ESHAPE): conv3d weights [Co, Ci, kt, kh, kw], conv2d weights
 *           [Co, Ci, kh, kw], biases [Co], RMS-norm gammas with C elements in any shape.
 *           The channel widths (decoder_base_dim) are taken from the shapes; anything
 *           other than the Wan2.2 layout (z_dim 48, widths 4b, 4b, 4b, 2b, b, 3 residual
 *           blocks per up block, temporal upsampling in up blocks 0 and 1, patch 2) is
 *           WANVAE_ETOPOLOGY. Duplicate names -> WANVAE_EARG.
 *  video    output [B, 3, 4T-3, 16h, 16w] NCTHW of element type dtype, values in [-1, 1]
 *           (NaN propagates).
 *  Requires B >= 1, T >= 1, h >= 1, w >= 1 and B * h * w <= 2^19. The decoder_base_dim b (the
 *  input channels of conv_out) must be 16, 32, 64, 96, 128 or 256 (the mid-block width 4b is
 *  one the attention kernels run: 64, 128, 256, 384, 512 or 1024), else WANVAE_ETOPOLOGY; this
 *  is checked with the other arguments, before anything is launched.
 */
int wanvae_decode_workspace_size(int64_t B, int64_t T, int64_t h, int64_t w,
                                 const wanvae_tensor *weights, int64_t n_weights,
                                 int32_t dtype, size_t *bytes);
int wanvae_decode(const void *z, int32_t z_dtype, int64_t B, int64_t T, int64_t h, int64_t w,
                  const wanvae_tensor *weights, int64_t n_weights, int32_t dtype,
                  void *video, void *workspace, size_t workspace_bytes, void *stream);

/*
 * wanvae_causal_conv3d -- one causal conv (WanCausalConv3d, "The parts": causal conv)
 * of a chunk x with n_cache frames of history:
 *   y[b,o,t,y,x] = bias[o] + sum_{i,dt,dy,dx} W[o,i,dt,dy,dx] * xt[b,i,t+dt,y+dy-kh/2,x+dx-kw/2]
 * where xt is (2*(kt/2) - n_cache) zero frames, then the cache frames, then x, with zero
 * padding kh/2, kw/2 in space. The sums accumulate in float32 ("Precision").
 *
 *  x        [B, Cin, t, h, w] (NCTHW) or [B, t, h, w, Cin] (NTHWC), element type dtype.
 *  cache    n_cache frames in the same layout ([B, Cin, n_cache, h, w] / [B, n_cache, h, w,
 *           Cin]), dtype; may be NULL when n_cache == 0. Requires 0 <= n_cache <= 2 and
 *           n_cache == 0 when kt == 1. In NTHWC both are read in place.
 *  weight   [Cout, Cin, kt, kh, kw] with kt in {1, 3}, kh, kw in {1, 3}; bias [Cout].
 *  y        [B, Cout, t, h, w] / [B, t, h, w, Cout] of element type y_dtype. y_dtype == dtype
 *           stores each sum + bias rounded to dtype; y_dtype = WANVAE_F32 with dtype =
 *           WANVAE_BF16 stores the float32 sum + bias unrounded. A float32 conv with a bf16
 *           y_dtype -> WANVAE_EDTYPE.
 *  cache_out  NULL, or the updated cache ("Causal caches": the last frames of cache ++ x):
 *           n_out = min(2, n_cache + t) frames, [B, Cin, n_out, h, w] / [B, n_out, h, w, Cin],
 *           dtype, written after y. It may be the cache buffer itself when n_cache == 2 (the
 *           in-place update); otherwise it must not overlap x, cache or y.
 *  Requires Cin a multiple of 8, Cout a multiple of 4, t <= 6, and x, cache, y, cache_out
 *  16-byte aligned (else WANVAE_EARG); y must not alias x or cache.
 *  Workspace: wanvae_causal_conv3d_workspace_size (its size bounds every kernel 1 <= kt*kh*kw
 *  <= 27 for Cout output channels).
 */
int wanvae_causal_conv3d_workspace_size(int64_t B, int64_t Cin, int64_t Cout, int64_t t, int64_t h,
                                        int64_t w, int64_t n_cache, int32_t layout, int32_t dtype,
                                        int32_t y_dtype, size_t *bytes);
int wanvae_causal_conv3d(const void *x, const void *cache, int64_t B, int64_t Cin, int64_t t,
                         int64_t h, int64_t w, int64_t n_cache, const wanvae_tensor *weight,
                         const wanvae_tensor *bias, int32_t layout, int32_t dtype, void *y,
                         int32_t y_dtype, void *cache_out, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * wanvae_causal_conv3d_noalloc -- wanvae_causal_conv3d for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid it). The
 * same conv, arguments, outputs and errors as wanvae_causal_conv3d, with its workspace in a
 * fixed 128 MiB device array of the library (one per GPU, held until the process ends)
 * instead of memory the call allocates or the caller brings; the call itself allocates
 * nothing. A conv whose workspace (wanvae_causal_conv3d_workspace_size) exceeds 128 MiB ->
 * WANVAE_EWORKSPACE before anything is launched (the 1024-channel 44 x 80 conv with two cached
 * frames takes 114 MB channels-last; channels-first layouts also hold converted copies of x,
 * cache and y). All calls on one GPU share its array: calls that overlap in time on one GPU
 * race, so the caller orders them (one stream, or events).
 */
int wanvae_causal_conv3d_noalloc(const void *x, const void *cache, int64_t B, int64_t Cin, int64_t t,
                                 int64_t h, int64_t w, int64_t n_cache, const wanvae_tensor *weight,
                                 const wanvae_tensor *bias, int32_t layout, int32_t dtype, void *y,
                                 int32_t y_dtype, void *cache_out, void *stream);

/*
 * wanvae_attn_block -- the mid-block attention block (WanAttentionBlock, "The parts":
 * attention), per frame of x [B, C, T, h, w]: n = RMS norm of x over channels (times
 * sqrt(C) and gamma); q, k, v = channels [0,C), [C,2C), [2C,3C) of a 1x1 conv C -> 3C
 * of n; O = softmax(q k^T / sqrt(C)) v over the h*w positions of the frame (one head of
 * dim C: the (N*T, H*W, 1, C) layout of MaxDiffusion PR #514's fix); y = proj(O) + x.
 *
 *  x       [B, C, T, h, w] (NCTHW) or [B, T, h, w, C] (NTHWC), dtype.
 *  gamma   C elements; qkv_w [3C, C, 1, 1] (or [3C, C]); qkv_b [3C];
 *          proj_w [C, C, 1, 1] (or [C, C]); proj_b [C].
 *  y       same shape and layout as x. Must not alias x.
 *  Requires C in {64, 128, 256, 384, 512, 1024} (the widths the attention kernels run),
 *  else WANVAE_ESHAPE.
 */
int wanvae_attn_block_workspace_size(int64_t B, int64_t C, int64_t T, int64_t h, int64_t w,
                                     int32_t layout, int32_t dtype, size_t *bytes);
int wanvae_attn_block(const void *x, int32_t layout, int64_t B, int64_t C, int64_t T, int64_t h,
                      int64_t w, const wanvae_tensor *gamma, const wanvae_tensor *qkv_w,
                      const wanvae_tensor *qkv_b, const wanvae_tensor *proj_w,
                      const wanvae_tensor *proj_b, int32_t dtype, void *y, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Kernel timing, for measurement. While enabled on a thread, every kernel the library
 * enqueues from that thread is bracketed by two HIP events recorded on the launch's stream,
 * and the launch's algorithmic work is noted: FLOPs of a conv (2 * outputs * Cin * kh * kw
 * * the time taps that fall on real frames; taps on a missing history frame are not
 * counted), FLOPs of the attention core (4 * S^2 * C per frame), bytes of a norm pass (its
 * input read once and output written once). wanvae_profile_enable(1) clears the records;
 * wanvae_profile_read(kind, ...) waits for the recorded events and returns, for the kernel
 * kind WANVAE_K*, the summed event time in ms, the launch count, and the summed FLOPs and
 * bytes. Any argument pointer may be NULL.
 */
#define WANVAE_KCONV 0
#define WANVAE_KNORM 1
#define WANVAE_KATTN 2
#define WANVAE_KOTHER 3
int wanvae_profile_enable(int on);
int wanvae_profile_read(int kind, double *ms, int64_t *launches, double *flops, double *bytes);

/*
 * Conv kernel selection, for testing and tuning. By default (kernel = -1) each conv takes the
 * kernel its shape and dtype call for. kernel in 0..WANVAE_CONV_KERNELS-1 asks every later
 * conv of any thread to use that kernel where it can run the conv (bf16 only for kernels 2
 * and 10..13; kernels 10, 12 and 13 only for 3x3 spatial convs with
 * Cin % 32 == 0 and Cout % 128 == 0, kernel 11 only for conv_out); other convs
 * keep the default. The kernels compute the same sums in different orders, so results agree
 * to rounding, not bit for bit. The environment variable WANVAE_CONV_TILE gives the initial
 * setting. Returns WANVAE_EARG for a kernel outside -1..WANVAE_CONV_KERNELS-1. Do not change
 * it while another thread is enqueueing work.
 *   0: 128 x 128 tile, register-staged loads    1: 32 x 256 (small Cout)
 *   2: 256 x 128, register-staged (bf16)         3..9: direct-to-LDS pipelines
 *  10: 3x3 halo tile, 128 channels x 16 x 32 positions, input patch shared by the taps (bf16)
 *  11: the same with 16 channels, for conv_out's unpatchify + clamp store (bf16)
 *  12: the 128-channel halo tile on 16 x 16 blocks (bf16)
 *  13: the 128-channel halo tile on 32 x 16 blocks (bf16)
 */
#define WANVAE_CONV_KERNELS 14
int wanvae_set_conv_kernel(int kernel);

/*
 * Norm kernel selection, for testing and tuning. In bf16 the SiLU after an RMS norm (the
 * residual blocks' norms and norm_out; page 3, "The parts" and "Precision") either runs as
 * arithmetic or reads a table of its bf16 results over the values of magnitude 2^-16 to 2^16,
 * built in each workgroup's LDS from the same arithmetic. Both give the same bits.
 *   mode -1 (default): the table on launches of at least 1,024 blocks of 16 waves, arithmetic
 *           on smaller ones; 0: arithmetic on every launch; 1: the table on every launch.
 * Applies to every later norm of any thread. The environment variable WANVAE_NORM_TAB gives the
 * initial setting. Returns WANVAE_EARG for a mode outside -1..1. Do not change it while another
 * thread is enqueueing work.
 */
int wanvae_set_norm_kernel(int mode);

/*
 * wanvae_decode_tiled -- the spatially tiled decode of the diffusers PR page "Implement tiled
 * VAE encoding/decoding for Wan model": the latent is cut into overlapping spatial tiles, each
 * decoded on its own as wanvae_decode does, and the decoded tiles are blended where they
 * overlap. It trades a different result for a workspace that scales with the tile, not the
 * video.
 *
 *  tile_h, tile_w, stride_h, stride_w  tile size and stride in VIDEO pixels (the page's defaults
 *           are 256 and 192), positive multiples of 16 with stride <= tile, else WANVAE_EARG.
 *           Tiles along an axis start at latent 0, s, 2s, ... (s = stride / 16) below the latent
 *           size and cover tile / 16 latents or what is left.
 *  Other arguments, the output and the errors are those of wanvae_decode.
 *
 * Composition (the blend rule is not on the page; this reading is the linear ramp diffusers'
 * VAEs use): in raster order, a decoded tile first takes a ramp with the tile above over its
 * first E_v = min(H_above, H, tile_h - stride_h) rows, row y becoming
 * above[H_above - E_v + y] * (1 - y/E_v) + own[y] * (y/E_v), then the same ramp with the tile
 * to its left over its first E_h columns, the neighbours as already composed; the weights are
 * float32 constants, and each product and the sum are rounded to dtype. The video takes rows
 * [0, stride_h) and columns [0, stride_w) of every composed tile.
 *
 * The tiles of one tile row with equal width are decoded as one batch. Workspace
 * (wanvae_decode_tiled_workspace_size): the rounded weights, two rows of decoded tiles, the
 * cropped latents of one batch and the decoder's buffers for one batch.
 */
int wanvae_decode_tiled_workspace_size(int64_t B, int64_t T, int64_t h, int64_t w, const wanvae_tensor *weights,
                                       int64_t n_weights, int32_t dtype, int32_t tile_h, int32_t tile_w,
                                       int32_t stride_h, int32_t stride_w, size_t *bytes);
int wanvae_decode_tiled(const void *z, int32_t z_dtype, int64_t B, int64_t T, int64_t h, int64_t w,
                        const wanvae_tensor *weights, int64_t n_weights, int32_t dtype, int32_t tile_h, int32_t tile_w,
                        int32_t stride_h, int32_t stride_w, void *video, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * Decode pipeline switch. With on = 1 (the default) wanvae_decode runs each latent frame's
 * work as two stages on two streams of its own (made once per device, default priority):
 * conv_in, the mid block and up block 0 of frame i+1 overlap up blocks 1-3 and conv_out of
 * frame i. This is the wavefront over the causal chunk loop that the page's chunked form
 * allows: a stage depends only on its own earlier chunks and on the stage before it of the
 * same chunk. Events order the stages; `stream` waits for both before the call's last
 * enqueued work, so the call stays ordered on `stream` as documented above. Every kernel
 * receives the same arguments either way, so the video is bit-identical with on = 0, which
 * runs everything on `stream` in chunk order. Decodes of one latent frame always run on
 * `stream`. Concurrent decodes on one device share the two streams and run one after the
 * other. Returns WANVAE_EARG for any value but 0 or 1. Do not change it while another thread
 * is enqueueing work.
 */
int wanvae_set_decode_pipeline(int on);

/* Message for the last failed call on this thread ("" if none). Valid until the next call. */
const char *wanvae_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int wanvae_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WANVAE_H */
