// Block-size selector for the fused forward.
//
// The pages choose tile sizes against on-chip memory capacity ("01 · 注意力为什么是
// IO 瓶颈", section 7, the block-size helper of the interface layer) and note that
// the gain depends on the number of compute units and the SRAM size (kp-015 page,
// "常见误区"). On gfx950 the limits are: 160 KB LDS per CU, 512 VGPR+AGPR per lane
// at one wave per SIMD, and 32x32x16 bf16 MFMA tiles.
//
// Two compiled shapes, both 4 waves with K/V tiles of 64 keys:
//  * BR = 256: each wave owns 64 query rows. Each wave reads every K/V tile from
//    LDS, so LDS bytes per MFMA flop fall as rows per wave rise; 64 rows keep the
//    K and V operand traffic (K by 128-bit reads, V by transposing 64-bit reads)
//    within the LDS read rate while the O accumulator (64 x d fp32) and Q (64 x d
//    bf16) stay in registers. One workgroup per CU (its four K/V stages of
//    2*64*d*2 bytes use 128 KB at d = 128; its registers allow one wave per SIMD).
//  * BR = 128: 32 rows per wave, twice the LDS operand traffic per flop, but half
//    the registers: two waves per SIMD, so at d = 64 (64 KB of stages) two
//    workgroups share a CU and one's softmax runs under the other's MFMAs.
// The selector estimates each shape's time as (rounds of resident workgroups) x
// (time of one round) and keeps the faster; ties keep 256. Round times relative
// to a round of 256-row workgroups, measured on one MI355X over 14 shapes:
//  * d = 128, one resident workgroup per CU either way: a 128-row round takes
//    0.59-0.60 of a 256-row round when both heights fill the chip. With twice the
//    rounds, 128 wins only where the 256-row grid's last round is at most about
//    half full (a grid of at most 128 tiles: measured 0.72-0.83 of the 256-row
//    time), and 256 everywhere else (128 measured 1.16-1.19 times slower).
//  * d = 64, two resident 128-row workgroups per CU: their round takes 0.93-1.0 of
//    a 256-row round, and with twice the workgroups and twice the residency the
//    round counts are equal, so 128 wins, by 25% when the 256-row grid leaves CUs
//    idle.

#include "fa_internal.h"

#include <algorithm>
#include <cstdint>

namespace fa {
namespace {

constexpr int kWaves = 4, kKeysPerTile = 64, kStages = 4;
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kCus = 256;  // MI355X; fixed so that a shape's results never depend on the device

constexpr int lds_bytes(int d) { return kStages * 2 * kKeysPerTile * d * 2; }
static_assert(lds_bytes(128) <= kLdsPerCu && lds_bytes(64) <= kLdsPerCu, "K/V ring must fit in LDS");

// Workgroups of one shape resident per CU: LDS-bound (1 or 2), and 1 for BR = 256
// (one wave per SIMD).
constexpr int resident(int d, int br) { return br == 256 ? 1 : (2 * lds_bytes(d) <= kLdsPerCu ? 2 : 1); }

}  // namespace

Blocks select_blocks(int d, int N, int B, int H) {
  Blocks b;
  b.nwaves = kWaves;
  b.bc = kKeysPerTile;
  b.br = 256;
  const int64_t bh = (int64_t)std::max(B, 0) * (int64_t)std::max(H, 0);
  const int64_t n = std::max(N, 1);
  // Time of a round of 128-row workgroups relative to a round of 256-row ones, in
  // thousandths.
  const int64_t rel128 = d == 64 ? 970 : 600;
  auto cost = [&](int br, int64_t rel) {
    const int64_t wgs = bh * ((n + br - 1) / br);
    const int64_t slots = (int64_t)kCus * resident(d, br);
    return (wgs + slots - 1) / slots * rel;
  };
  if (bh > 0 && cost(128, rel128) < cost(256, 1000)) b.br = 128;
  return b;
}

// Split of the key range for the decode-shaped forward (few query rows, long K/V).
// Each (b, h) is cut into S chunks of `chunk` keys, one workgroup per chunk. The
// split kernel streams K and V; the grid aims at kCus times a per-kernel count of
// workgroups per CU. For the matrix-core kernel (2 to 16 rows) that count is what
// its registers let a CU hold at d = 128 (254 VGPRs: 2 workgroups of 4 waves); at
// d = 64 it takes 140 VGPRs (3 workgroups) and the count is 4. For the vector
// kernel of one query row (90 VGPRs: 5 workgroups) the count is 7: a grid of more
// workgroups than fit at once keeps more loads in flight while the first ones
// drain, and planning for 7 measured faster than planning for 5 (6768-6799 against
// 6431-6450 GB/s at B=16 H=32 Nk=8192 d=128, 4 against 3 chunks per head). More,
// shorter chunks add partial
// results to write and merge. Chunks hold at least 256 keys and are multiples of
// 128 keys, a whole number of the kernel's key batches for both head dimensions.
// Depends on the shape only, not on the device.
namespace {
int resident_per_cu(int Nq, int d) { return Nq <= 1 ? 7 : d == 64 ? 4 : 2; }
}  // namespace

DecodePlan decode_plan(int B, int H, int Nq, int Nk, int d) {
  constexpr int64_t kMinChunk = 256, kAlign = 128;
  const int64_t target = (int64_t)kCus * resident_per_cu(Nq, d);
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
