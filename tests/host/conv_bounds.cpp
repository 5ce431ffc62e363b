// Host-side checks of the conv kernels' launch conditions (run by tests/test_host_cpp.py,
// linked against libwanvae.so; no GPU needed: nothing is launched).
//
// The halo-tile conv addresses one input frame of one batch element with 32-bit byte offsets
// and marks the padding with the offset 2^31, so it must refuse frames of 2^31 bytes or more
// (those take the implicit-GEMM kernel, which addresses in 64 bits). Prints one line per case:
// "<name> <0|1>".
#include <cstdio>

#include "internal.h"

using namespace wanvae;

static void report(const char* name, int Hin, int Win, int Cin, int Cout, int up, int tile, int mode) {
  ConvArgs a{};
  a.kt = up ? 1 : 3;
  a.kh = a.kw = 3;
  a.Cin = Cin, a.Cout = Cout;
  a.Hin = Hin, a.Win = Win;
  a.up = up;
  a.Ho = up ? 2 * Hin : Hin, a.Wo = up ? 2 * Win : Win;
  a.B = 1, a.F = 4;
  a.mode = mode;
  printf("%s %d\n", name, conv_halo_supported(a, kBF16, tile) ? 1 : 0);
}

int main() {
  // level 3 of a 2208 x 3840 video (latent 138 x 240): up_blocks.3.resnets.0.conv1 reads 512
  // channels of 1104 x 1920 = 2,170,552,320 bytes > 2^31
  report("l3_512_138x240", 1104, 1920, 512, 256, 0, kTileHalo128x16x32, kEpiFrames);
  // a 2160 x 3840 video (latent 135 x 240): 1080 x 1920 x 512 x 2 = 2,123,366,400 bytes < 2^31
  report("l3_512_135x240", 1080, 1920, 512, 256, 0, kTileHalo128x16x32, kEpiFrames);
  // the 256-channel convs of the same level: half the bytes
  report("l3_256_138x240", 1104, 1920, 256, 256, 0, kTileHalo128x16x32, kEpiFrames);
  // exactly 2^31 bytes: refused (offset 2^31 is the padding marker)
  report("exact_2p31", 1024, 2048, 512, 256, 0, kTileHalo128x16x32, kEpiFrames);
  report("below_2p31", 1024, 2047, 512, 256, 0, kTileHalo128x16x32, kEpiFrames);
  // the upsampling conv reads the low-resolution frame: its bytes count
  report("up_l2_to_l3_138x240", 552, 960, 512, 512, 1, kTileHalo128x16x32, kEpiFrames);
  // conv_out's 16-channel tile and the float32-output epilogue follow the same bound
  report("conv_out_138x240", 1104, 1920, 256, 12, 0, kTileHalo16x16x32, kEpiVideo);
  report("f32_out_704x1280", 352, 640, 256, 256, 0, kTileHalo128x16x32, kEpiFramesF32);
  report("video_epilogue_on_128_tile", 352, 640, 256, 256, 0, kTileHalo128x16x32, kEpiVideo);
  return 0;
}
