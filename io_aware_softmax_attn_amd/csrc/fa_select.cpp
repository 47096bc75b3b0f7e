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

#include <algorithm>
#include <cstdint>

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

// Split of the key range for the decode-shaped forward (few query rows, long K/V).
// Each (b, h) is cut into S chunks of `chunk` keys, one workgroup per chunk. The
// split kernel streams K and V, so the grid aims at one full round of resident
// workgroups: 256 CUs times the workgroups one CU holds at once, which the kernel's
// register use sets per compiled row count (70, 80, 110, 170 and 256 VGPRs for up
// to 1, 2, 4, 8 and 16 query rows: 7, 6, 4, 2 and 1 workgroups of 4 waves). A
// second, partial round would leave most CUs idle at the end; more, shorter chunks
// add partial results to write and merge. Chunks hold at least 256 keys and are
// multiples of 128 keys, a whole number of the kernel's key batches for both head
// dimensions. Depends on the shape only, not on the device.
namespace {
constexpr int kCus = 256;
int resident_per_cu(int Nq) { return Nq <= 1 ? 7 : Nq <= 2 ? 6 : Nq <= 4 ? 4 : Nq <= 8 ? 2 : 1; }
}  // namespace

DecodePlan decode_plan(int B, int H, int Nq, int Nk, int d) {
  (void)d;
  constexpr int64_t kMinChunk = 256, kAlign = 128;
  const int64_t target = (int64_t)kCus * resident_per_cu(Nq);
  const int64_t bh = std::max<int64_t>(1, (int64_t)B * H);
  const int64_t nk = std::max<int64_t>(1, Nk);
  int64_t s = (target + bh - 1) / bh;
  s = std::max<int64_t>(1, std::min(s, (nk + kMinChunk - 1) / kMinChunk));
  int64_t chunk = (nk + s - 1) / s;
  chunk = std::min(nk, (chunk + kAlign - 1) / kAlign * kAlign);
  DecodePlan p;
  p.splits = (int)((nk + chunk - 1) / chunk);
  p.chunk = (int)chunk;
  return p;
}

}  // namespace fa
