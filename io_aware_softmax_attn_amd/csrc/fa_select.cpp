// Block-size selector for the fused forward.
//
// The pages choose tile sizes against on-chip memory capacity ("01 · 注意力为什么是
// IO 瓶颈", section 7, the block-size helper of the interface layer) and note that
// the gain depends on the number of compute units and the SRAM size (kp-015 page,
// "常见误区"). On gfx950 the limits are: 160 KB LDS per CU, 512 VGPR+AGPR per lane
// at one wave per SIMD, and 32x32x16 bf16 MFMA tiles.
//
// Shape used for both head dimensions: 4 waves, each owning 64 query rows
// (BR = 256), K/V tiles of 64 keys. Each wave reads every K/V tile from LDS, so
// LDS bytes per MFMA flop fall as rows per wave rise; 64 rows keep the K and V
// operand traffic (K by 128-bit reads, V by transposing 64-bit reads) within the
// LDS read rate while the O accumulator (64 x d fp32) and Q (64 x d bf16) stay in
// registers. Four K/V stages of 2*64*d*2 bytes use 128 KB at d = 128.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4, kRowsPerWave = 64, kKeysPerTile = 64, kStages = 4;
constexpr int kLdsPerCu = 160 * 1024;

constexpr int lds_bytes(int d) { return kStages * 2 * kKeysPerTile * d * 2; }
static_assert(lds_bytes(128) <= kLdsPerCu && lds_bytes(64) <= kLdsPerCu, "K/V ring must fit in LDS");

}  // namespace

Blocks select_blocks(int d, int N, int B, int H) {
  (void)d;
  (void)N;
  (void)B;
  (void)H;
  Blocks b;
  b.nwaves = kWaves;
  b.br = kWaves * kRowsPerWave;
  b.bc = kKeysPerTile;
  return b;
}

}  // namespace fa
