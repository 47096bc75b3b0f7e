// Fused attention forward for gfx950 (MI355X): O = softmax(scale * Q K^T) V and
// the per-row natural-log LSE, in one kernel that never writes S or P to memory.
//
// Method ("Flash Attention (FA1)" page: "Tiling in FlashAttention", "Online
// Softmax in FlashAttention" and the update derivation, steps 1-5; "01 · 注意力为什么
// 是 IO 瓶颈" page, section 5 skeleton: query tiles outer, K/V tiles streamed inner):
// each workgroup owns one tile of BR query rows of one (b, h) and streams every
// K/V tile of that head through LDS, keeping per row a running reference max m,
// a running sum l of exp2 terms and an unnormalised output accumulator; O and
// LSE = ln2 * (m + log2 l) are written once at the end.
//
// gfx950 design (not the pages' GPU design):
//  * Transposed products. The kernel computes S^T = K Q^T and O^T = V^T P^T with
//    v_mfma_f32_32x32x16_bf16 so that each lane holds one query column: row max
//    and row sum are in-lane reductions plus one permlane32 swap, and the S^T
//    accumulator converts in registers (v_cvt_pk_bf16_f32) straight into the B
//    operand of the PV product; P never leaves VGPRs.
//  * The key order inside a 32-key block is permuted (row bits 2 and 3 swapped
//    when K rows are fed to the MFMA) so that the accumulator layout of S^T
//    matches the operand layout that ds_read_b64_tr_b16 produces for V^T. The
//    contraction over keys does not depend on key order.
//  * 4 waves x 64 query rows per workgroup (BR = 256), or x 32 rows (BR = 128,
//    for grids that 256-row tiles would leave partly idle, and for d = 64, where
//    two such workgroups share a CU); 64-key K/V tiles, four
//    LDS stages filled by direct global->LDS 16-byte loads (buffer_load_dwordx4
//    ... lds, through per-tile buffer resources that read rows past N as zero)
//    with a XOR swizzle of 16-byte chunks against LDS bank conflicts.
//  * Software pipeline over 32-key sub-tiles: while the matrix cores run the PV
//    product of sub-tile j-1 and the scores of j+1, the VALU runs the softmax of j,
//    one score register per MFMA slot. The main loop is unrolled over the 8-step
//    period of the LDS ring, so every LDS offset is an instruction immediate.
//  * exp2 with log2(e) folded into the score scale. The exp2 terms are formed
//    against the current reference max without a per-tile max; the reference
//    moves (and the accumulator is rescaled) only when a row's terms over a
//    sub-tile sum past 2^16. Any reference gives the same O and LSE in exact
//    arithmetic; O is divided by the sum of the bf16-rounded terms that built the
//    accumulator (computed on the matrix cores), so the weights applied to V sum
//    to one whatever the reference.
//  * Workgroup ids are remapped so that each XCD (8 per chip, dispatched
//    round-robin) runs consecutive query tiles of the same head, keeping that
//    head's K/V hot in the XCD's L2.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// K/V tiling, common to both query-tile heights. A wave owns NQB blocks of 32
// query rows (NQB = 2: BR = 256 rows per workgroup; NQB = 1: BR = 128).
template <int D>
struct Cfg {
  static constexpr int kWaves = 4;
  static constexpr int kBC = 64;
  static constexpr int kStages = 4;     // K/V tiles resident in LDS
  static constexpr int kAhead = kStages - 2;  // tiles loading while the current one is read
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;  // 16-byte chunks per K/V row
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;  // K tile, then V tile
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kLoadsPerTile = kTileBytes / 1024;  // one load = 64 lanes x 16 B
  static constexpr int kLoadsPerWave = kLoadsPerTile / kWaves;
  static constexpr int kKS = D / 16;  // 16-wide k-steps of the QK^T contraction
  static constexpr int kDB = D / 32;  // 32-wide blocks of d in O^T
  // Offsets from the LDS base of 32-key sub-tile jj's K rows and V rows (jj >= 0;
  // the stage ring has a period of 2 * kStages sub-tiles).
  static constexpr int k_tile_off(int jj) { return ((jj >> 1) % kStages) * kStageBytes + (jj & 1) * 32 * kRowBytes; }
  static constexpr int v_tile_off(int jj) { return k_tile_off(jj) + kTileBytes; }
  static_assert(kLoadsPerTile % kWaves == 0, "tile loads must split evenly over waves");
};

// XOR swizzle of the 16-byte chunk index by row (bits 0-3 only, so 16-row-aligned
// sub-tile bases keep it). With 64 banks of 4 bytes an LDS cycle serves 256 bytes:
//  * a ds_read_b128 quarter-wave reads one logical chunk of 16 different rows; the
//    swizzle is a bijection on the row's low bits, so the 16 reads land in 16
//    distinct 16-byte slots of the bank line;
//  * a ds_read_b64_tr_b16 half-wave reads 4 consecutive rows x 4 chunks (two lane
//    groups of 16 with chunk bit 1 = 0 and 1); the swizzle varies with the row
//    only in chunk bits 2-3 (d = 128) or bit 2 and the bank-line half (d = 64), so
//    the two groups fill disjoint halves and the half-wave covers every slot once.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

template <int D>
__device__ __forceinline__ int chunk_offset(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ swz<D>(row)) << 4);
}

// MFMA row rho of a 32-key block reads key pi(rho): bits 2 and 3 swapped.
__device__ __forceinline__ int pi_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Workgroup id -> logical tile id such that XCD x (ids w with w % 8 == x) gets a
// contiguous range of logical ids.
__device__ __forceinline__ int remap_xcd(int w, int total) {
  const int xcd = w & 7, idx = w >> 3;
  const int base = total >> 3, rem = total & 7;
  return xcd < rem ? xcd * (base + 1) + idx : rem * (base + 1) + (xcd - rem) * base + idx;
}

// Logical tile id (bh * tiles_per_head + query tile) of workgroup w under a tile
// order (the orders of fa_fwd_tile_order): 0 keeps each head's tiles on one XCD;
// 1 takes them in dispatch order, so the dispatcher deals a head's consecutive
// tiles to all 8 XCDs; 2 runs query-tile-major (consecutive workgroups belong to
// different heads), so the tiles of one head are spread over time and XCDs.
__device__ __forceinline__ int tile_of(int w, int total, int tiles_per_head, int order) {
  if (order == 1) return w;
  if (order == 2) {
    const int bhs = total / tiles_per_head;
    return (w % bhs) * tiles_per_head + w / bhs;
  }
  return remap_xcd(w, total);
}

// v_permlane32_swap with both operands = x: lanes 0-31 receive lanes 32-63 in one
// result and vice versa, so max/sum of the two results reduces over lanes l, l^32.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for the K/V pipeline: each wave has waited for its own
// direct-to-LDS loads (vmcnt), so after s_barrier every wave's share of the tile is
// in LDS. LDS reads still in flight target stages nobody overwrites here, so no
// lgkmcnt wait is needed (unlike __syncthreads). The asm memory clobbers keep the
// compiler from moving LDS accesses across the barrier.
template <int kOutstanding>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(kOutstanding >= 0 && kOutstanding <= 63, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOutstanding) : "memory");
}

// kOutstanding: this wave's loads of later tiles that may stay in flight (loads
// complete in issue order, so everything older, i.e. the tile about to be read,
// has landed).
template <int kOutstanding>
__device__ __forceinline__ void tile_barrier() {
  wait_vmcnt<kOutstanding>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte offset, within a K or V tile in global memory, of the 16 bytes that lane
// `lane` of wave `wave` copies with its i-th direct-to-LDS load. Slot p (16 bytes,
// lane-consecutive per instruction) holds row p / kChunks and physical chunk
// p % kChunks, i.e. logical chunk (p % kChunks) ^ swz(row).
template <int D>
__device__ __forceinline__ unsigned tile_load_offset(int wave, int lane, int i, int* row_out) {
  using C = Cfg<D>;
  const int p = (wave * C::kLoadsPerWave + i) * 64 + lane;
  const int row = p / C::kChunks;
  const int chunk = (p % C::kChunks) ^ swz<D>(row);
  *row_out = row;
  return (unsigned)(row * (D * 2) + chunk * 16);
}

// Buffer resource over the part of K or V tile u of one head (head = that head's
// base) that lies inside N: at most one tile, none for tiles past the end. A
// buffer load outside it returns zeros without touching memory, so the ragged
// last tile and the loads issued past the last tile need no clamping and no
// branch. Word 3 selects raw 32-bit data (no swizzle, no index stride).
// Words: base address bits 0-31, bits 32-47 (stride 0), size in bytes, format.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr unsigned kRawBufferWord3 = 0x00020000u;
template <int D>
__device__ __forceinline__ u32x4_t tile_rsrc(const char* head, int u, int N) {
  using C = Cfg<D>;
  const int rows = min(max(N - u * C::kBC, 0), C::kBC);
  const uint64_t base = (uint64_t)(uintptr_t)head + (uint64_t)u * C::kTileBytes;
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)base);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(base >> 32) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane((unsigned)(rows * C::kRowBytes));
  r[3] = kRawBufferWord3;
  return r;
}

// One 16-byte-per-lane direct global->LDS load (buffer_load_dwordx4 ... lds):
// lane l's 16 bytes, at byte offset voff of the resource, land at LDS address
// lds_addr + 16*l. Issued through asm so that the compiler, which cannot tell that
// the destination stage is disjoint from the stages being read, does not put a
// vmcnt(0) wait in front of the next LDS read; the pipeline waits for these loads
// itself (tile_barrier). M0 carries the LDS address (one wait state between its
// write and the load).
__device__ __forceinline__ void dma16(u32x4_t rsrc, unsigned voff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Issue this wave's loads of K tile u (kV = false) or V tile u (kV = true) of one
// head into `stage`. gofs holds this lane's tile_load_offset values.
template <int D, bool kV>
__device__ __forceinline__ void issue_half(const char* __restrict__ head, int u, int N, unsigned stage, int wave,
                                           const unsigned* gofs) {
  using C = Cfg<D>;
  const u32x4_t r = tile_rsrc<D>(head, u, N);
  const unsigned dst = __builtin_amdgcn_readfirstlane(stage + (kV ? C::kTileBytes : 0) +
                                                      (unsigned)(wave * C::kLoadsPerWave * 1024));
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) dma16(r, gofs[i], dst + i * 1024);
}

// ---------------------------------------------------------------------------
// MFMA issue with pinned register classes. The scores S^T live in VGPRs (the
// softmax reads them with VALU instructions); the output accumulator O^T lives
// in AGPRs for the whole kernel (only MFMAs and the rare rescale touch it). The
// compiler does not see these as MFMAs, so the code below keeps the required
// wait states itself: S is first read by VALU code after the next step's first
// MFMA (see the slot-0 s_nop in pipeline_step), P is written at least one step
// before the MFMA that reads it, and every VALU access to O^T goes through
// sync_acc() first.
// Scores: the Q^T operand (b) stays in AGPRs too, as the MFMA B source.
__device__ __forceinline__ void mfma_s(f32x16_t& d, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s0(f32x16_t& d, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_o(f32x16_t& d, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Row sums of a P^T operand: v_mfma_f32_16x16x32_bf16 with a 0/1 selector as A.
// Read as the B operand of this instruction, lane l of a P^T fragment holds 8 of
// the 32 k-values of column l%16: k-group l/16, which is keys 0-7 of query l%32
// for lanes 0-31 and keys 8-15 of query l%32 for lanes 32-63. The selector makes
// output rows 0-7 sum k-groups 0 and 2 (query n) and rows 8-15 k-groups 1 and 3
// (query n+16), so lane l of the result holds the full 16-key sum of query
// (l%16) + 16*(l/32), in all four of its registers. Products with 0 and 1 are
// exact and the sum is fp32, so this is the sum of the bf16 terms the PV product
// used. The selector is tied as read-write so the compiler keeps it in place
// instead of rewriting it (with a VALU move) in front of every use; the s_nop
// covers the two wait states a VALU write needs before an MFMA reads it, should
// the compiler ever move it anyway.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void mfma_rowsum(f32x4_t& d, bf16x8_t& sel, const bf16x8_t& p) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d), "+v"(sel) : "v"(p));
}

// Wait states between the last MFMA that wrote an accumulator and VALU reads of it.
__device__ __forceinline__ void sync_acc(f32x16_t& a, f32x16_t& b) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+a"(a), "+a"(b));
}
__device__ __forceinline__ void sync_acc(f32x16_t& a) { asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+a"(a)); }
template <int DB, int NQB>
__device__ __forceinline__ void sync_acc_all(f32x16_t (&acc)[DB][NQB]) {
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    if constexpr (NQB == 2) {
      sync_acc(acc[db][0], acc[db][1]);
    } else {
      sync_acc(acc[db][0]);
    }
  }
}

// Key index, within a 32-key sub-tile, of S^T accumulator register i, minus 8g:
// key = 8g + 16*(i/8) + 4*((i/4)%2) + i%4 (the pi row permutation).
__device__ __forceinline__ constexpr int key_of_reg(int i) { return 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3); }

template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

// State of one wave's 32*NQB query rows (32-row MFMA column blocks qb < NQB).
template <int D, int NQB>
struct Wave {
  using C = Cfg<D>;
  bf16x8_t qf[NQB][C::kKS];   // Q^T operands (AGPRs)
  unsigned koff[C::kKS];      // LDS addresses of this lane's K operand reads (stage 0, sub-tile 0)
  unsigned voff[C::kDB][2];   // ... and of its V transposing reads (tile base excluded)
  unsigned koff2[C::kKS];     // the same plus 64 KiB: bases for sub-tiles whose offset exceeds
  unsigned voff2[C::kDB][2];  // the 16-bit immediate of ds_read
  unsigned gofs[C::kLoadsPerWave];  // this lane's tile_load_offset values
  f32x16_t acc[C::kDB][NQB];  // O^T accumulator (AGPRs)
  float m[NQB];               // reference max, log2 units
  float l[NQB];               // this lane's part of the running sum of the exp2 terms (for LSE)
  f32x4_t lbacc[NQB];         // row sums of the bf16 terms that entered the PV product (for O)
  bf16x8_t sel;               // the 0/1 selector operand of mfma_rowsum
  bf16x8_t vpre[4];           // V^T operands of the next step's first PV slots, read ahead
  bool rescale;               // the reference max moved in the last softmax: scale acc
  float alpha[NQB];           // ... by exp2(m_old - m_new) before the next PV product
};

// Online-softmax reference update for one 32-key sub-tile (FA1 page, derivation
// steps 1-2), the slow path: the row max of the sub-tile's scaled scores, a new
// reference max m_new = max(m, rowmax) per row, alpha = exp2(m_old - m_new), and l
// rescaled. The max is taken over the scaled scores s * c, so that it is the max
// of the softmax's arguments for a scale of either sign. kMasked leaves keys >=
// nvalid (passed as nvalid - 8g) out of the max; the caller's exp2 stage zeroes
// their terms.
template <bool kMasked, int NQB>
__device__ __forceinline__ void move_reference(const f32x16_t (&s)[NQB], float (&m)[NQB], float (&l)[NQB],
                                               float (&alpha)[NQB], float c, int nv8) {
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float x = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float t = s[qb][i] * c;
      if constexpr (kMasked) {
        if (key_of_reg(i) >= nv8) t = -__builtin_inff();
      }
      x = fmaxf(x, t);
    }
    const float mn = fmaxf(m[qb], pair_max(x));
    alpha[qb] = __builtin_amdgcn_exp2f(m[qb] - mn);
    m[qb] = mn;
    l[qb] *= alpha[qb];
  }
}

// One pipeline step j over 32-key sub-tiles (FA1 page, derivation steps 1-5, with
// the division by l deferred to the end). The matrix cores add sub-tile j-1's PV
// product (kPV) and then compute the scores of sub-tile j+1 (kQK), while the VALU
// does the online softmax of sub-tile j (kExp: scores in scur, exp2 terms into
// pcur), so no MFMA depends on a VALU result of the same step.
//
// Softmax: the exp2 terms are formed against the current reference max m without
// computing the tile max first (the reference starts at sub-tile 0's row max). If
// some row's sum of terms over the sub-tile exceeds 2^16, the wave takes a slow
// path that moves the reference to the row max (move_reference), schedules the
// accumulator rescale for the next step and recomputes the terms.
// Otherwise every term is at most 2^16, far inside fp32 and bf16 range, and in
// exact arithmetic the result does not depend on the reference. In rounded
// arithmetic the terms' bf16 rounding does; dividing O by the sum of the rounded
// terms (lb) rather than of the exact ones cancels it for the terms that dominate
// a row, whatever the reference. The work is staged over the step's PV and score
// MFMA slots: slot s issues the fma of about one score register, the exp2 of those
// of slot s-1 and the sum and bf16 packing of those of slot s-2, so no instruction
// waits for one issued in the same slot. scur and snxt are different registers (the scores of j+1 are written while
// those of j are read). kMasked: sub-tile j is the ragged last one (keys >= nvalid,
// passed as nvalid - 8g, are masked). kJP >= 0: j mod the ring period (2 * kStages)
// is known at compile time.
template <int D, int NQB, bool kPV, bool kExp, bool kQK, bool kMasked, int kJP>
__device__ __forceinline__ void pipeline_step(Wave<D, NQB>& w, int j, int T, int N, const char* gk, const char* gv,
                                              LDS_AS char* lds, int wave, int lane, f32x16_t (&scur)[NQB],
                                              f32x16_t (&snxt)[NQB], const bf16x8_t (&pprev)[NQB][2],
                                              bf16x8_t (&pcur)[NQB][2], float c, int nv8) {
  using C = Cfg<D>;
  constexpr int KS = C::kKS, DB = C::kDB;
  constexpr int NPV = kPV ? 2 * DB * NQB : 0;     // MFMA slots of the PV product (first)
  constexpr int NS = NPV + (kQK ? KS * NQB : 0);  // all MFMA slots
  constexpr int NE = 16 * NQB;                    // score registers per lane (NQB blocks x 16)
  // The softmax is staged over the NS MFMA slots: NAS slots issue fma work, exp2
  // and packing trail by one and two slots. Each PV slot whose d-block is 1 is
  // followed by a row-sum MFMA of the same P^T operand (16x16x32, half as long),
  // which carries no softmax work of its own. The softmax ends kCheckLead slots
  // before the step does: the reference-move test is taken there and branched on
  // only after the last MFMA, so its dependence chain (last exp2, sums, compare,
  // ballot) resolves under MFMAs.
  constexpr int kCheckLead = NS >= 12 ? 2 : 0;
  constexpr int NAS = NS >= 3 + kCheckLead ? NS - 2 - kCheckLead : 0;
  constexpr int NPAIR = 2 * DB;                // V^T operand pairs (h, db) of a PV product
  constexpr int kVPre = 4;                     // pairs read in the previous step
  constexpr int kVLead = 4;                    // other pairs: read this many pairs ahead
  // K operand reads run four k-steps (4 * NQB slots) ahead of their MFMA, starting
  // kKStart slots in; with fewer PV slots, three are read before the first slot.
  constexpr int kKLead = 4 * NQB;
  constexpr int kKStart = NPV > kKLead ? NPV - kKLead : 0;
  constexpr float kSumLimit = 65536.0f;
  static_assert(NPAIR >= kVPre, "prefetch depth");

  if constexpr (kPV) {
    // The previous softmax moved the reference max (uniform branch, rarely
    // taken): bring the PV products accumulated so far to the new reference.
    if (__builtin_expect(w.rescale, false)) {
      sync_acc_all(w.acc);
      // One fragment at a time: each asm ties the finished fragment to the next
      // one, so the compiler cannot pull all of them into VGPRs at once.
#pragma unroll
      for (int f = 0; f < NQB * DB; ++f) {
        w.acc[f / NQB][f % NQB] *= w.alpha[f % NQB];
        if (f + 1 < NQB * DB)
          asm volatile("" : "+a"(w.acc[f / NQB][f % NQB]), "+a"(w.acc[(f + 1) / NQB][(f + 1) % NQB]));
      }
      // The row-sum MFMAs of the previous step finished during sync_acc's wait; the
      // empty asm keeps the reads below after it. Lane l's row sum belongs to query
      // (l%16) + 16*(l/32) (see mfma_rowsum), whose alpha sits in lane (that query).
      if constexpr (NQB == 2) {
        asm volatile("" : "+v"(w.lbacc[0]), "+v"(w.lbacc[1]));
      } else {
        asm volatile("" : "+v"(w.lbacc[0]));
      }
      const int src = ((lane & 15) | ((lane >> 5) << 4)) * 4;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        w.lbacc[qb] *= __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, w.alpha[qb])));
      if constexpr (NQB == 2) {
        asm volatile("s_nop 1" : "+v"(w.lbacc[0]), "+v"(w.lbacc[1]));
      } else {
        asm volatile("s_nop 1" : "+v"(w.lbacc[0]));
      }
      sync_acc_all(w.acc);
      w.rescale = false;
    }
  }
  // kJP >= 0: j mod the ring period is known at compile time, and with it every LDS
  // offset below.
  const bool odd = kJP >= 0 ? (kJP & 1) != 0 : (j & 1) != 0;
  if constexpr (kQK) {
    if (odd) {  // sub-tile j+1 opens K/V tile t: wait for it
      static_assert(C::kAhead >= 1 && C::kAhead <= 3, "wait counts below cover up to two later tiles");
      constexpr int kPerTile = 2 * C::kLoadsPerWave;  // this wave's loads per K/V tile
      const int t = (j + 1) >> 1;
      // Tiles t+1 .. t+kAhead-1 (those that exist) may stay in flight.
      const int later = min(C::kAhead - 1, T - 1 - t);
      if (later >= 2) {
        tile_barrier<2 * kPerTile>();
      } else if (later == 1) {
        tile_barrier<kPerTile>();
      } else {
        tile_barrier<0>();
      }
    }
  }
  // Loads of K/V tile u = t + kAhead, spread over the MFMA slots of the two steps of
  // tile t: the step that opens it (j odd) loads u's K tile, the next one its V tile.
  // Stage u % kStages last held tile u - kStages = t - 2, whose final operand reads
  // completed in step 2t - 2, before the barrier above.
  // Past the last tile the resource is empty and the loads only zero a free stage.
  const int u_dma = ((j + 1) >> 1) + C::kAhead;
  const bool dma_v = !odd;
  const u32x4_t dma_rsrc = tile_rsrc<D>(dma_v ? gv : gk, u_dma, N);
  const int dma_stage = kJP >= 0 ? (((kJP + 1) >> 1) + C::kAhead) % C::kStages : u_dma % C::kStages;
  const unsigned dma_dst = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)lds + (unsigned)(dma_stage * C::kStageBytes + (dma_v ? C::kTileBytes : 0) +
                                           wave * C::kLoadsPerWave * 1024));
  __builtin_amdgcn_sched_barrier(0);

  // Byte offsets (uniform, SGPR) of this step's sub-tiles from the LDS base: K of
  // j+1, V of j-1, and V of j (read ahead for the next step). readfirstlane: one
  // scalar value each, so every operand address is one v_add.
  // This step's sub-tiles: K of j+1, V of j-1, V of j (read ahead for the next
  // step). Scalars when j % 8 is not known at compile time: one v_add per read.
  const unsigned kst = __builtin_amdgcn_readfirstlane(kQK ? (unsigned)C::k_tile_off(j + 1) : 0u);
  const unsigned vst = __builtin_amdgcn_readfirstlane(kPV ? (unsigned)C::v_tile_off(j - 1) : 0u);
  const unsigned vnx = __builtin_amdgcn_readfirstlane(kExp ? (unsigned)C::v_tile_off(j) : 0u);
  constexpr int kKOff = kJP >= 0 ? C::k_tile_off(kJP + 1) : 0;
  constexpr int kVOff = kJP >= 0 ? C::v_tile_off(kJP + 2 * C::kStages - 1) : 0;  // j - 1 (mod the period)
  constexpr int kVNxOff = kJP >= 0 ? C::v_tile_off(kJP) : 0;

  // V^T operand pair pr of the sub-tile at offset `off` (constant) or `base` (scalar).
  auto read_v = [&](auto off_tag, unsigned base, int pr) -> bf16x8_t {
    constexpr int off = decltype(off_tag)::value;
    const int h = pr / DB, db = pr % DB;
    unsigned a0, a1;
    if constexpr (kJP >= 0) {
      // Folded into the 16-bit immediate; the second base set covers offsets past 64 KiB.
      if (off + h * 16 * C::kRowBytes >= 65536) {
        a0 = w.voff2[db][0] + (off + h * 16 * C::kRowBytes - 65536);
        a1 = w.voff2[db][1] + (off + h * 16 * C::kRowBytes - 65536);
      } else {
        a0 = w.voff[db][0] + (off + h * 16 * C::kRowBytes);
        a1 = w.voff[db][1] + (off + h * 16 * C::kRowBytes);
      }
    } else {
      const unsigned b = base + h * 16 * C::kRowBytes;
      a0 = w.voff[db][0] + b;
      a1 = w.voff[db][1] + b;
    }
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(uintptr_t)a0);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(uintptr_t)a1);
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4,
                                   5, 6, 7);
  };
  bf16x8_t kf[KS];
  bf16x8_t vf[NPAIR];
  auto load_k = [&](auto ks_tag) {
    constexpr int ks = decltype(ks_tag)::value;
    if constexpr (kQK && ks < KS) {
      unsigned a;
      if constexpr (kJP < 0) {
        a = w.koff[ks] + kst;
      } else if constexpr (kKOff >= 65536) {
        a = w.koff2[ks] + (kKOff - 65536);
      } else {
        a = w.koff[ks] + kKOff;
      }
      kf[ks] = *(const LDS_AS bf16x8_t*)(uintptr_t)a;
    }
  };
  auto load_v = [&](auto p_tag) {
    constexpr int p = decltype(p_tag)::value;
    if constexpr (kPV && p >= kVPre && p < NPAIR) vf[p] = read_v(std::integral_constant<int, kVOff>{}, vst, p);
  };
  auto prefetch_next = [&](auto p_tag) {
    constexpr int p = decltype(p_tag)::value;
    if constexpr (kExp && p < kVPre) w.vpre[p] = read_v(std::integral_constant<int, kVNxOff>{}, vnx, p);
  };
  if constexpr (kPV) {
#pragma unroll
    for (int p = 0; p < kVPre; ++p) vf[p] = w.vpre[p];
  }


  // ---- softmax of sub-tile j, staged: fma (A), exp2 (B), sum + pack (C) ----
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  float tv[NQB][16];
  float sum[NQB][2];  // per-lane partial sums of the terms, even and odd registers
  unsigned pk[NQB][8];  // packed bf16 pairs, assembled into pcur per 8-key operand
  auto stage_a = [&](auto e_tag) {
    constexpr int e = decltype(e_tag)::value, qb = e / 16, i = e % 16;
    tv[qb][i] = __builtin_fmaf(scur[qb][i], c, -w.m[qb]);
  };
  auto stage_b = [&](auto e_tag) {
    constexpr int e = decltype(e_tag)::value, qb = e / 16, i = e % 16;
    float pe = __builtin_amdgcn_exp2f(tv[qb][i]);
    if constexpr (kMasked) {
      if (key_of_reg(i) >= nv8) pe = 0.0f;
    }
    tv[qb][i] = pe;
  };
  auto stage_c = [&](auto e_tag) {
    constexpr int e = decltype(e_tag)::value, qb = e / 16, i = e % 16;
    // The first term of each partial sum is assigned, not added to 0: the compiler
    // may not fold 0 + x (x = -0 would differ), and the terms are never -0.
    if constexpr (i < 2) {
      sum[qb][i] = tv[qb][i];
    } else {
      sum[qb][i & 1] += tv[qb][i];
    }
    if constexpr (i & 1) {  // registers i-1, i -> one packed bf16 pair (v_cvt_pk_bf16_f32, nearest-even)
      const bf16x2_t pr = __builtin_convertvector((f32x2_t){tv[qb][i - 1], tv[qb][i]}, bf16x2_t);
      pk[qb][i >> 1] = __builtin_bit_cast(unsigned, pr);
      if constexpr ((i & 7) == 7) {  // a whole 8-key operand: assemble it once
        constexpr int f = i >> 3;
        pcur[qb][f] = __builtin_bit_cast(
            bf16x8_t, (u32x4_t){pk[qb][4 * f], pk[qb][4 * f + 1], pk[qb][4 * f + 2], pk[qb][4 * f + 3]});
      }
    }
  };
  // Elements whose fma is issued in slot s (s < NAS); exp2 in s+1, pack in s+2.
  auto a_begin = [](int s) constexpr { return (s * NE) / (NAS > 0 ? NAS : 1); };
  auto softmax_slot = [&](auto s_tag) {
    constexpr int s = decltype(s_tag)::value;
    // Pin the values entering this slot's fma and exp2 work to the slot start:
    // scores not yet scaled and scaled scores awaiting exp2. Without these the
    // instruction scheduler may hoist work of later slots into earlier ones,
    // overloading those slots. Empty asm: no instructions. (exp2 results are not
    // pinned: the compiler guards an asm that reads a transcendental's result with
    // an s_nop, and the packing after them is pinned at its end anyway.)
    {
      auto& tvw = tv;  // named here: asm operands alone do not capture in a generic lambda
      auto& sw = scur;
      if constexpr (s == 0) {
        // First VALU read of the scores: after slot 0's MFMA, which cannot issue
        // before the previous step's last MFMA has run its 32 cycles, so the MFMAs
        // that wrote scur (issued before that one) have finished. The s_nop adds the
        // two wait states of a VALU read after an MFMA issue.
        // With one column block the last MFMA of the previous step wrote scur itself;
        // it still ran before slot 0's MFMA could issue.
        if constexpr (NQB == 2) {
          asm volatile("s_nop 1" : "+v"(sw[0]), "+v"(sw[1]));
        } else {
          asm volatile("s_nop 1" : "+v"(sw[0]));
        }
      } else if constexpr (s < NAS && a_begin(s) < 16) {
        asm volatile("" : "+v"(sw[0]));
      }
      if constexpr (NQB == 2 && s < NAS && a_begin(s + 1) > 16) asm volatile("" : "+v"(sw[NQB - 1]));
      if constexpr (s >= 1) {
#pragma unroll
        for (int e = a_begin(s - 1); e < a_begin(s); ++e) asm volatile("" : "+v"(tvw[e >> 4][e & 15]));
      }
    }
    if constexpr (s < NAS) static_for<a_begin(s), a_begin(s + 1)>(stage_a);
    if constexpr (s >= 1 && s - 1 < NAS) static_for<a_begin(s - 1), a_begin(s)>(stage_b);
    if constexpr (s >= 2 && s - 2 < NAS) {
      static_for<a_begin(s - 2), a_begin(s - 1)>(stage_c);
      // Pin the packed words this slot produced to the slot, so later passes cannot
      // sink the softmax past it. Single registers: pinning a partly built
      // 4-register operand would make the compiler copy it.
      auto& pkw = pk;  // named here: asm operands alone do not capture in a generic lambda
#pragma unroll
      for (int e = a_begin(s - 2) | 1; e < a_begin(s - 1); e += 2) asm volatile("" : "+v"(pkw[e >> 4][(e & 15) >> 1]));
    }
  };
  // Taken after the step's last MFMA (see check_softmax): the slow path if some
  // row's terms grew too large.
  uint64_t big_rows = 0;  // ballot of rows whose terms grew too large
  auto check_softmax = [&]() {
    if constexpr (kExp) {
      bool big = sum[0][0] + sum[0][1] > kSumLimit;
      if constexpr (NQB == 2) big = big || (sum[1][0] + sum[1][1] > kSumLimit);
      big_rows = __builtin_amdgcn_ballot_w64(big);
    }
  };
  auto finish_softmax = [&]() {
    if constexpr (kExp) {
      if (__builtin_expect(big_rows != 0, false)) {
        float alpha[NQB];
        move_reference<kMasked>(scur, w.m, w.l, alpha, c, nv8);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) w.alpha[qb] = alpha[qb];
        w.rescale = kPV;  // before the first PV product acc is zero: nothing to rescale
        static_for<0, NE>(stage_a);
        static_for<0, NE>(stage_b);
        static_for<0, NE>(stage_c);
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) w.l[qb] += sum[qb][0] + sum[qb][1];
    }
  };

  // Reads issued before the first slot.
  static_for<0, NPAIR>([&](auto p_tag) {
    constexpr int p = decltype(p_tag)::value;
    if constexpr (NQB * (p - kVLead) < 0) load_v(p_tag);
  });
  if constexpr (kKStart == 0) static_for<0, 3>(load_k);
  if constexpr (kExp && NAS == 0) {  // too few slots to carry the softmax: do it before any MFMA
    static_for<0, NE>(stage_a);
    static_for<0, NE>(stage_b);
    static_for<0, NE>(stage_c);
    check_softmax();
  }

  // PV slots whose d-block is 1 are followed by the row-sum MFMA of their P^T operand.
  auto rowsum_after = [](int s) constexpr { return s < NPV && (s / NQB) % DB == 1; };
  // Two waves per SIMD (d = 64, 128-row tiles): a wave raises its issue priority
  // over its score slots, which the SIMD's arbitration otherwise shares evenly
  // with the other wave (measured at B=1 H=32 N=8192: kernel cycles -6.6%, matrix
  // cores 0.605 busy against 0.565; over the PV slots instead: -1.5%).
  constexpr bool kPrio = D == 64 && NQB == 1 && kQK;
  static_for<0, NS>([&](auto s_tag) {
    constexpr int s = decltype(s_tag)::value;
    if constexpr (kPrio && s == NPV) __builtin_amdgcn_s_setprio(1);
    if constexpr (s < NPV) {
      constexpr int pr = s / NQB, qb = s % NQB;
      constexpr int h = pr / DB, db = pr % DB;
      mfma_o(w.acc[db][qb], vf[pr], pprev[qb][h]);
      // V pairs kVLead pairs ahead of their first slot.
      static_for<0, NPAIR>([&](auto p_tag) {
        constexpr int p = decltype(p_tag)::value;
        if constexpr (NQB * (p - kVLead) == s) load_v(p_tag);
      });
    } else {
      constexpr int ks = (s - NPV) / NQB, qb = (s - NPV) % NQB;
      if constexpr (ks == 0) {
        mfma_s0(snxt[qb], kf[ks], w.qf[qb][ks]);
      } else {
        mfma_s(snxt[qb], kf[ks], w.qf[qb][ks]);
      }
      // read ahead the next step's first V pairs
      if constexpr (qb == NQB - 1 && ks < kVPre) prefetch_next(std::integral_constant<int, ks>{});
    }
    // K operand reads, starting kKStart slots in.
    if constexpr (kQK && s >= kKStart && (s - kKStart) % NQB == 0) {
      constexpr int n = (s - kKStart) / NQB;  // n-th K read of this step, needed at slot NPV + NQB*n
      if constexpr (kKStart > 0) {
        load_k(std::integral_constant<int, n>{});
      } else {
        load_k(std::integral_constant<int, n + 3>{});
      }
    }
    if constexpr (kQK) {
      constexpr int L = C::kLoadsPerWave, every = NS / L;
      if constexpr (s % every == 1 && s / every < L) {
        constexpr int i = s / every;
        dma16(dma_rsrc, w.gofs[i], dma_dst + i * 1024);
      }
    }
    if constexpr (kExp && NAS > 0) {
      softmax_slot(std::integral_constant<int, s>{});
      if constexpr (s == NAS + 1) check_softmax();
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (rowsum_after(s)) {
      constexpr int qb = s % NQB, h = (s / NQB) / DB;
      mfma_rowsum(w.lbacc[qb], w.sel, pprev[qb][h]);
      __builtin_amdgcn_sched_barrier(0);
    }
  });
  if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
  if constexpr (kExp && !kQK) {  // no score slots: read the next step's V operands now
    static_for<0, kVPre>(prefetch_next);
  }
  __builtin_amdgcn_sched_barrier(0);
  // After the last MFMA: the slow path if some row's terms grew too large.
  finish_softmax();
}

// NQB = 2: 256 query rows per workgroup, one wave per SIMD. NQB = 1: 128 rows
// per workgroup; at d = 64 its registers allow two waves per SIMD and two
// workgroups' K/V rings fit in LDS, so two workgroups share a CU. (At d = 128 the
// 128 KB ring allows one workgroup per CU whatever the registers.)
template <int D, int NQB>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(D == 64 ? 3 - NQB : 1, D == 64 ? 3 - NQB : 1)))
fa_fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
              __bf16* __restrict__ o, float* __restrict__ lse, int N, int tiles_per_head, int total_tiles,
              float c /* scale * log2(e) */, int order) {
  using C = Cfg<D>;
  constexpr int kRowsPerWave = 32 * NQB;
  constexpr int kBR = C::kWaves * kRowsPerWave;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];
  // The LDS base as a scalar: every LDS address below is a scalar offset plus at
  // most one per-lane term.
  LDS_AS char* lds = (LDS_AS char*)(uintptr_t)__builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(LDS_AS char*)smem);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;  // which half of the wave
  const int logical = tile_of(blockIdx.x, total_tiles, tiles_per_head, order);
  const int bh = logical / tiles_per_head;
  const int qtile = logical - bh * tiles_per_head;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const char* gk = (const char*)(k + head_off);
  const char* gv = (const char*)(v + head_off);
  const int T = (N + C::kBC - 1) / C::kBC;  // K/V tiles in LDS
  const int U = (N + 31) / 32;              // 32-key sub-tiles processed by the pipeline
  const int q0 = qtile * kBR + wave * kRowsPerWave;

  Wave<D, NQB> w;
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    int row;
    w.gofs[i] = tile_load_offset<D>(wave, lane, i, &row);
  }
  // Start streaming K/V tile 0 while Q is loaded.
  const unsigned lds_u = (unsigned)(uintptr_t)lds;
  issue_half<D, false>(gk, 0, N, lds_u, wave, w.gofs);
  issue_half<D, true>(gv, 0, N, lds_u, wave, w.gofs);

  // Q^T operand fragments: lane holds query q0 + qb*32 + lane%32, d = ks*16 + g*8 .. +8.
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = q0 + qb * 32 + (lane & 31);
    const bf16x8_t* src = (const bf16x8_t*)(q + head_off + (size_t)min(row, N - 1) * D + g * 8);
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      bf16x8_t xq = src[ks * 2];
      if (row >= N) xq = bf16x8_t{};
      w.qf[qb][ks] = xq;
    }
  }
  // Wait states between the AGPR writes of Q^T and the first MFMA that reads them.
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    if constexpr (NQB == 2) {
      asm volatile("s_nop 1" : "+a"(w.qf[0][ks]), "+a"(w.qf[1][ks]));
    } else {
      asm volatile("s_nop 1" : "+a"(w.qf[0][ks]));
    }
  }
  asm volatile("s_nop 7" ::: "memory");
  // Per-lane LDS byte offsets of the operand reads (sub-tile base added later; the
  // swizzle depends on row bits 0-3 only, so 16-row-aligned bases keep it).
  const unsigned lds_base = (unsigned)(uintptr_t)lds;
  {
    const int r0 = pi_row(lane & 31);
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      w.koff[ks] = lds_base + chunk_offset<D>(r0, ks * 2 + g);
      w.koff2[ks] = w.koff[ks] + 65536u;
      // Opaque to the compiler, which would otherwise recompute it per read.
      asm volatile("" : "+v"(w.koff2[ks]));
    }
  }
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 8 * g + 4 * r + ((lane & 15) >> 2);
      const int dcol = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      w.voff[db][r] = lds_base + chunk_offset<D>(row, dcol >> 3) + 2 * (dcol & 7);
      w.voff2[db][r] = w.voff[db][r] + 65536u;
      asm volatile("" : "+v"(w.voff2[db][r]));
    }
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    w.m[qb] = -__builtin_inff();
    w.l[qb] = 0.0f;
    w.lbacc[qb] = f32x4_t{};
  }
  {
    // Selector: lane l holds row l%16 of k-group l/16; 1 where rows 0-7 meet
    // k-groups 0, 2 and rows 8-15 meet k-groups 1, 3.
    const bool one = ((lane & 15) < 8) == (((lane >> 4) & 1) == 0);
    const unsigned word = one ? 0x3F803F80u : 0u;  // two bf16 1.0 or two zeros
    w.sel = __builtin_bit_cast(bf16x8_t, (u32x4_t){word, word, word, word});
  }
  w.rescale = false;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) w.alpha[qb] = 1.0f;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) w.acc[db][qb] = f32x16_t{};
  }

  wait_vmem();
  __syncthreads();
  // Tiles 1 .. kAhead-1 and the K half of tile kAhead; from step 0 on each step
  // loads one half of a later tile.
#pragma unroll
  for (int t = 1; t <= C::kAhead; ++t) {
    if (t < T) {
      issue_half<D, false>(gk, t, N, lds_u + t * C::kStageBytes, wave, w.gofs);
      if (t < C::kAhead) issue_half<D, true>(gv, t, N, lds_u + t * C::kStageBytes, wave, w.gofs);
    }
  }

  const int nvalid_last = N - (U - 1) * 32;  // 1..32 keys in the last sub-tile
  const bool ragged = nvalid_last < 32;
  const int nv8 = nvalid_last - 8 * g;
  f32x16_t sa[NQB], sb[NQB];
  bf16x8_t pa[NQB][2], pb[NQB][2];

  // Scores of sub-tile 0.
  {
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      const bf16x8_t kfr = *(const LDS_AS bf16x8_t*)(uintptr_t)w.koff[ks];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        if (ks == 0) {
          mfma_s0(sa[qb], kfr, w.qf[qb][ks]);
        } else {
          mfma_s(sa[qb], kfr, w.qf[qb][ks]);
        }
      }
    }
    if constexpr (NQB == 2) {
      asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+v"(sa[0]), "+v"(sa[1]));
    } else {
      asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+v"(sa[0]));
    }
  }
  // The reference max starts at sub-tile 0's row max (move_reference from m = -inf:
  // alpha = 0 and l stays 0), so the first softmax step takes the fast path.
  {
    float alpha0[NQB];
    if (U == 1 && ragged) move_reference<true>(sa, w.m, w.l, alpha0, c, nv8);
    else move_reference<false>(sa, w.m, w.l, alpha0, c, nv8);
  }

  // Step j: PV of j-1, softmax of j, scores of j+1. Two score buffers alternate,
  // so the softmax of j can spread over every MFMA slot of the step.
#define FA_STEPP(JP, PV, EXP, QK, MASK, J, SC, SN, PP, PC) \
  pipeline_step<D, NQB, PV, EXP, QK, MASK, JP>(w, J, T, N, gk, gv, lds, wave, lane, SC, SN, PP, PC, c, nv8)
#define FA_STEP(PV, EXP, QK, MASK, J, SC, SN, PP, PC) FA_STEPP(-1, PV, EXP, QK, MASK, J, SC, SN, PP, PC)
  if (U == 1) {
    if (ragged) FA_STEP(false, true, false, true, 0, sa, sb, pb, pa);
    else FA_STEP(false, true, false, false, 0, sa, sb, pb, pa);
  } else {
    FA_STEP(false, true, true, false, 0, sa, sb, pb, pa);
  }
  // Full steps j = 1 .. U-2: one period of the LDS stage ring (2 * kStages steps)
  // per iteration while they last (j = 1 mod the period there, so every LDS offset
  // is a compile-time constant), then two at a time.
  constexpr int kPeriod = 2 * C::kStages;
  int j = 1;
  for (; j + kPeriod - 1 <= U - 2; j += kPeriod) {
    static_for<0, kPeriod>([&](auto i_tag) {
      constexpr int i = decltype(i_tag)::value;  // step j + i; odd when i is even
      if constexpr (i % 2 == 0) {
        FA_STEPP((i + 1) % kPeriod, true, true, true, false, j + i, sb, sa, pa, pb);
      } else {
        FA_STEPP((i + 1) % kPeriod, true, true, true, false, j + i, sa, sb, pb, pa);
      }
    });
  }
  for (; j + 1 <= U - 2; j += 2) {
    FA_STEP(true, true, true, false, j, sb, sa, pa, pb);
    FA_STEP(true, true, true, false, j + 1, sa, sb, pb, pa);
  }
  if (j <= U - 2) {  // one more full step, j odd
    FA_STEP(true, true, true, false, j, sb, sa, pa, pb);
    ++j;
  }
  // j == U - 1 when U >= 2: PV of U-2 and softmax of the last sub-tile; then step U:
  // PV of the last sub-tile.
  if (U >= 2) {
    if (j & 1) {
      if (ragged) FA_STEP(true, true, false, true, j, sb, sa, pa, pb);
      else FA_STEP(true, true, false, false, j, sb, sa, pa, pb);
      FA_STEP(true, false, false, false, j + 1, sa, sb, pb, pa);
    } else {
      if (ragged) FA_STEP(true, true, false, true, j, sa, sb, pb, pa);
      else FA_STEP(true, true, false, false, j, sa, sb, pb, pa);
      FA_STEP(true, false, false, false, j + 1, sb, sa, pa, pb);
    }
  } else {
    FA_STEP(true, false, false, false, 1, sb, sa, pa, pb);
  }
#undef FA_STEP
#undef FA_STEPP

  // Loads issued after the last tile barrier (zero fills past the last tile) must
  // land before the workgroup's LDS can be handed to another workgroup.
  wait_vmem();

  // Epilogue: O = acc / lb (bf16, nearest-even), LSE = ln2 * (m + log2 l). O is
  // divided by the sum of the bf16-rounded terms that formed acc, so the weights
  // it applies to V sum to one exactly; LSE takes the sum of the unrounded terms.
  sync_acc_all(w.acc);
  // read after sync_acc's wait
  if constexpr (NQB == 2) {
    asm volatile("" : "+v"(w.lbacc[0]), "+v"(w.lbacc[1]));
  } else {
    asm volatile("" : "+v"(w.lbacc[0]));
  }
  // The rounded-term sum of query q (this lane's q = lane%32) sits in lane q for
  // q < 16 and lane q + 16 otherwise (see mfma_rowsum).
  const int q32 = lane & 31;
  const int lb_src = (q32 < 16 ? q32 : q32 + 16) * 4;
  // O goes through LDS: each lane holds 8-byte pieces of 32 different rows, so
  // storing it directly would take 32 scattered stores per lane. Written into a
  // row-major tile of this wave's rows (row pitch padded by 16 bytes against
  // bank conflicts) and read back by rows, it leaves as fully coalesced 16-byte
  // stores (16 per lane at 64 rows per wave and d = 128). The K/V stages are idle by then: the barrier waits until every
  // wave has finished its last step (and, with the vmem wait above, every load).
  __syncthreads();
  constexpr int kOPitch = D * 2 + 16;
  static_assert(C::kWaves * kRowsPerWave * kOPitch <= C::kLdsBytes, "O staging tiles must fit in the K/V stages");
  const unsigned otile = (unsigned)(uintptr_t)lds + (unsigned)(wave * kRowsPerWave * kOPitch);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lsum = pair_sum(w.l[qb]);
    const float lbq = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(lb_src, __builtin_bit_cast(int, w.lbacc[qb][0])));
    const float inv = 1.0f / lbq;
    const unsigned rbase = otile + (unsigned)((qb * 32 + (lane & 31)) * kOPitch + 8 * g);
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4_t wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = (__bf16)(w.acc[db][qb][i4 * 4 + e] * inv);
        *(LDS_AS bf16x4_t*)(uintptr_t)(rbase + (unsigned)((db * 32 + 8 * i4) * 2)) = wv;
      }
    }
    const int row = q0 + qb * 32 + (lane & 31);
    if (g == 0 && row < N) lse[(size_t)bh * N + row] = kLn2 * (w.m[qb] + log2f(lsum));
  }
  // Read back by rows: 16-byte chunk c = lane + 64*k is row c / kChunks, chunk c % kChunks.
  constexpr int kRowsPerPass = 64 / C::kChunks;
#pragma unroll
  for (int k = 0; k < kRowsPerWave / kRowsPerPass; ++k) {
    const int r = k * kRowsPerPass + lane / C::kChunks, ch = lane % C::kChunks;
    const bf16x8_t x = *(const LDS_AS bf16x8_t*)(uintptr_t)(otile + (unsigned)(r * kOPitch + ch * 16));
    const int row = q0 + r;
    if (row < N) *(bf16x8_t*)(o + head_off + (size_t)row * D + ch * 8) = x;
  }
}

}  // namespace

int device_is_gfx950() {
  // Cached per device: 0 unknown, 1 gfx950, 2 other.
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    const int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (c != 0) return c == 1 ? 1 : 0;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_HIP;
  const char* a = prop.gcnArchName;
  const int is950 = (a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' && a[5] == '0') ? 1 : 0;
  if (dev >= 0 && dev < 64) __atomic_store_n(&cache[dev], is950 ? 1 : 2, __ATOMIC_RELAXED);
  return is950;
}

int launch_fused(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                 float scale, const Blocks& blk, void* stream, int order) {
  // The compiled shapes: 4 waves, 64-key K/V tiles, 256 or 128 query rows.
  if (blk.nwaves != 4 || blk.bc != 64 || (blk.br != 256 && blk.br != 128)) return FA_ERR_SHAPE;
  const int tiles = (N + blk.br - 1) / blk.br;
  const long long total = (long long)B * H * tiles;
  const float c = scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
#define FA_LAUNCH(D, NQB)                                                                                        \
  hipLaunchKernelGGL((fa_fwd_kernel<D, NQB>), dim3((unsigned)total), dim3(256), 0, s, (const __bf16*)q,           \
                     (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, N, tiles, (int)total, c, order)
  if (d == 128) {
    if (blk.br == 256) FA_LAUNCH(128, 2);
    else FA_LAUNCH(128, 1);
  } else {
    if (blk.br == 256) FA_LAUNCH(64, 2);
    else FA_LAUNCH(64, 1);
  }
#undef FA_LAUNCH
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
