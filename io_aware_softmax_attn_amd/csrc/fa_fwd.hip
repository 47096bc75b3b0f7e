// Fused attention forward for gfx950 (MI355X): O = softmax(scale * Q K^T) V and
// the per-row natural-log LSE, in one kernel that never writes S or P to memory.
//
// Method ("Flash Attention (FA1)" page: "Tiling in FlashAttention", "Online
// Softmax in FlashAttention" and the update derivation, steps 1-5; "01 · 注意力为什么
// 是 IO 瓶颈" page, section 5 skeleton: query tiles outer, K/V tiles streamed inner):
// each workgroup owns one tile of BR query rows of one (b, h) and streams every
// K/V tile of that head through LDS, keeping per row a running reference max m,
// a running sum l of exp2 terms and an unnormalised output accumulator; O = acc/l
// and LSE = ln2 * (m + log2 l) are written once at the end.
//
// gfx950 design (not the pages' GPU design):
//  * Transposed products. The kernel computes S^T = K Q^T and O^T = V^T P^T with
//    v_mfma_f32_32x32x16_bf16 so that each lane holds one query column: the row
//    max and row sum are in-lane reductions plus one permlane32 swap, and the
//    S^T accumulator converts in registers (v_cvt_pk_bf16_f32) straight into the
//    B operand of the PV product; P never leaves VGPRs.
//  * The key order inside a 32-key block is permuted (row bits 2 and 3 swapped
//    when K rows are fed to the MFMA) so that the accumulator layout of S^T
//    matches the operand layout that ds_read_b64_tr_b16 produces for V^T. The
//    contraction over keys does not depend on key order.
//  * 4 waves x 64 query rows per workgroup (BR = 256), 64-key K/V tiles, three
//    LDS stages filled by direct global->LDS 16-byte loads (global_load_lds_dwordx4)
//    with a XOR swizzle of 16-byte chunks against LDS bank conflicts.
//  * exp2 with log2(e) folded into the score scale; the rescale of the
//    accumulator is skipped while the tile max stays within 2^8 of the reference
//    max (any reference gives the same O and LSE; only the magnitude of the exp2
//    terms depends on it).
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
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Rescale the accumulator only when a tile's max exceeds the reference by more
// than this (log2 units); exp2 terms then stay <= 2^8, far from fp32/bf16 limits.
constexpr float kRescaleThreshold = 8.0f;

template <int D>
struct Cfg {
  static constexpr int kWaves = 4;
  static constexpr int kRowsPerWave = 64;
  static constexpr int kBR = kWaves * kRowsPerWave;
  static constexpr int kBC = 64;
  static constexpr int kStages = 3;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;  // 16-byte chunks per K/V row
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;  // K tile, then V tile
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kLoadsPerTile = kTileBytes / 1024;  // one load = 64 lanes x 16 B
  static constexpr int kLoadsPerWave = kLoadsPerTile / kWaves;
  static constexpr int kKS = D / 16;  // 16-wide k-steps of the QK^T contraction
  static constexpr int kDB = D / 32;  // 32-wide blocks of d in O^T
  static_assert(kLoadsPerTile % kWaves == 0, "tile loads must split evenly over waves");
};

// XOR swizzle of the 16-byte chunk index by row, so that the 16 lanes of one
// ds_read_b128 (16 rows, same chunk) and the 16 lanes of one ds_read_b64_tr_b16
// (4 consecutive rows x 2 chunks) hit distinct bank groups.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return ((row & 7) << 1) | ((row >> 3) & 1);
  } else {
    return (row & 6) | ((row >> 3) & 1);
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

// Issue the direct-to-LDS loads of K and V tile t of one head into `stage`.
// Slot p (16 bytes, lane-consecutive per instruction) holds row p / kChunks and
// physical chunk p % kChunks, i.e. logical chunk (p % kChunks) ^ swz(row). Rows
// past N re-read row N-1: finite data whose scores are masked to -inf.
template <int D>
__device__ __forceinline__ void issue_tile(const char* __restrict__ gk, const char* __restrict__ gv, int t, int N,
                                           LDS_AS char* stage, int wave, int lane) {
  using C = Cfg<D>;
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    const int ii = wave * C::kLoadsPerWave + i;
    const int p = ii * 64 + lane;
    const int row = p / C::kChunks;
    const int chunk = (p % C::kChunks) ^ swz<D>(row);
    const int grow = min(t * C::kBC + row, N - 1);
    const size_t goff = (size_t)grow * (D * 2) + (size_t)chunk * 16;
    __builtin_amdgcn_global_load_lds(gk + goff, (LDS_AS void*)(stage + ii * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gv + goff, (LDS_AS void*)(stage + C::kTileBytes + ii * 1024), 16, 0, 0);
  }
}

// Scores of one 32-key sub-tile: S^T[qb] = K_sub Q_block(qb)^T over all of d.
// kst points at the sub-tile's first key row in LDS.
template <int D>
__device__ __forceinline__ void qk_sub(f32x16_t (&s)[2], const bf16x8_t (&qf)[2][Cfg<D>::kKS],
                                       const LDS_AS char* kst, const int (&koff)[Cfg<D>::kKS]) {
  using C = Cfg<D>;
  s[0] = f32x16_t{};
  s[1] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    const bf16x8_t a = *(const LDS_AS bf16x8_t*)(kst + koff[ks]);
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][ks], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[1][ks], s[1], 0, 0, 0);
  }
}

// Key index, within a 32-key sub-tile, of S^T accumulator register i, minus 8g:
// key = 8g + 16*(i/8) + 4*((i/4)%2) + i%4 (the pi row permutation).
__device__ __forceinline__ constexpr int key_of_reg(int i) { return 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3); }

// Online-softmax part 1 on one sub-tile (FA1 page, derivation steps 1-2): the row
// max of the sub-tile, and a new reference max where it exceeds the current one
// by more than the threshold. Returns whether any row of the wave moved its
// reference; then alpha = exp2(m_old - m_new) and l has been scaled by it (the
// caller scales acc once the previous sub-tile's PV product is in). kMasked sets
// keys >= nvalid (passed as nvalid - 8g) to -inf.
template <bool kMasked>
__device__ __forceinline__ bool sub_max(f32x16_t (&s)[2], float (&m)[2], float (&l)[2], float (&alpha)[2], float c,
                                        int nvalid_minus_8g) {
  float mt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float x = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (kMasked) {
        if (key_of_reg(i) >= nvalid_minus_8g) s[qb][i] = -__builtin_inff();
      }
      x = fmaxf(x, s[qb][i]);
    }
    mt[qb] = pair_max(x) * c;
  }
  const bool need = (mt[0] > m[0] + kRescaleThreshold) || (mt[1] > m[1] + kRescaleThreshold);
  const bool any = __builtin_amdgcn_ballot_w64(need) != 0;
  if (any) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mn = fmaxf(m[qb], mt[qb]);
      alpha[qb] = __builtin_amdgcn_exp2f(m[qb] - mn);
      m[qb] = mn;
      l[qb] *= alpha[qb];
    }
  }
  return any;
}

// Online-softmax part 2 (FA1 page, step 1 numerators, step 2 running sum):
// P~ = exp2(s*c - m) in fp32, l += rowsum(P~), and P~ rounded to bf16 in the
// B-operand layout of the PV product: p[qb][h] holds accumulator registers 8h..8h+7.
template <bool kMasked>
__device__ __forceinline__ void sub_exp(const f32x16_t (&s)[2], const float (&m)[2], float (&l)[2],
                                        bf16x8_t (&p)[2][2], float c, int nvalid_minus_8g) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float negm = -m[qb];
    float sum = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8_t v;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = h * 8 + j;
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][i], c, negm));
        if constexpr (kMasked) {
          if (key_of_reg(i) >= nvalid_minus_8g) e = 0.0f;
        }
        sum += e;
        v[j] = (__bf16)e;
      }
      p[qb][h] = v;
    }
    l[qb] += sum;
  }
}

// acc^T[db][qb] += V_sub^T(db) P^T(qb) for one 32-key sub-tile (two 16-key steps).
// vst points at the sub-tile's first value row in LDS.
template <int D>
__device__ __forceinline__ void pv_sub(f32x16_t (&acc)[Cfg<D>::kDB][2], const bf16x8_t (&p)[2][2],
                                       const LDS_AS char* vst, const int (&voff)[Cfg<D>::kDB][2]) {
  using C = Cfg<D>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
      const LDS_AS char* base = vst + h * 16 * C::kRowBytes;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(base + voff[db][0]));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(base + voff[db][1]));
      const bf16x8_t a = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
      acc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[0][h], acc[db][0], 0, 0, 0);
      acc[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[1][h], acc[db][1], 0, 0, 0);
    }
  }
}

// acc *= alpha, in place in AGPRs, when flag != 0. VALU cannot read AGPRs, so each
// element goes through a VGPR. The branch lives inside the asm so that the
// compiler sees one unconditional definition of acc and keeps it in the same
// AGPRs across the loop. The s_nops cover the wait states after the MFMA that
// last wrote acc and before the next MFMA reads it.
__device__ __forceinline__ void scale_agpr_if(f32x16_t& a, float alpha, unsigned flag) {
  float t;
  asm volatile(
      "s_cmp_eq_u32 %18, 0\n\t"
      "s_cbranch_scc1 .Lskip_scale%=\n\t"
      "s_nop 15\n\ts_nop 15\n\ts_nop 15\n\t"
      "v_accvgpr_read_b32 %16, %0\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %0, %16\n\t"
      "v_accvgpr_read_b32 %16, %1\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %1, %16\n\t"
      "v_accvgpr_read_b32 %16, %2\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %2, %16\n\t"
      "v_accvgpr_read_b32 %16, %3\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %3, %16\n\t"
      "v_accvgpr_read_b32 %16, %4\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %4, %16\n\t"
      "v_accvgpr_read_b32 %16, %5\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %5, %16\n\t"
      "v_accvgpr_read_b32 %16, %6\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %6, %16\n\t"
      "v_accvgpr_read_b32 %16, %7\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %7, %16\n\t"
      "v_accvgpr_read_b32 %16, %8\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %8, %16\n\t"
      "v_accvgpr_read_b32 %16, %9\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %9, %16\n\t"
      "v_accvgpr_read_b32 %16, %10\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %10, %16\n\t"
      "v_accvgpr_read_b32 %16, %11\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %11, %16\n\t"
      "v_accvgpr_read_b32 %16, %12\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %12, %16\n\t"
      "v_accvgpr_read_b32 %16, %13\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %13, %16\n\t"
      "v_accvgpr_read_b32 %16, %14\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %14, %16\n\t"
      "v_accvgpr_read_b32 %16, %15\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %15, %16\n\t"
      "s_nop 7\n"
      ".Lskip_scale%=:"
      : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(a[4]), "+a"(a[5]), "+a"(a[6]), "+a"(a[7]),
        "+a"(a[8]), "+a"(a[9]), "+a"(a[10]), "+a"(a[11]), "+a"(a[12]), "+a"(a[13]), "+a"(a[14]), "+a"(a[15]),
        "=&v"(t)
      : "v"(alpha), "s"(flag)
      : "scc");
}

// One software-pipeline step over 32-key sub-tiles: the PV product of sub-tile u
// (P operand cur) overlaps the scores and exp2 terms of sub-tile u+1 (into nxt).
// When sub-tile u+1 starts a new K/V tile, wait for its loads, synchronise the
// workgroup and start loading the following tile into the stage that the tile
// before u's has freed. kMasked: sub-tile u+1 is the ragged last one.
template <int D, bool kMasked>
__device__ __forceinline__ void pipeline_step(int u, int T, int N, const char* gk, const char* gv, LDS_AS char* lds,
                                              int wave, int lane, f32x16_t (&s)[2],
                                              const bf16x8_t (&qf)[2][Cfg<D>::kKS], const int (&koff)[Cfg<D>::kKS],
                                              const int (&voff)[Cfg<D>::kDB][2], float (&m)[2], float (&l)[2],
                                              f32x16_t (&acc)[Cfg<D>::kDB][2], const bf16x8_t (&cur)[2][2],
                                              bf16x8_t (&nxt)[2][2], float c, int nv8) {
  using C = Cfg<D>;
  if (u & 1) {
    const int t = (u + 1) >> 1;
    wait_vmem();
    __syncthreads();
    if (t + 1 < T) issue_tile<D>(gk, gv, t + 1, N, lds + ((t + 1) % C::kStages) * C::kStageBytes, wave, lane);
  }
  const int un = u + 1;
  qk_sub<D>(s, qf, lds + ((un >> 1) % C::kStages) * C::kStageBytes + (un & 1) * 32 * C::kRowBytes, koff);
  float alpha[2] = {1.0f, 1.0f};
  const bool rescale = sub_max<kMasked>(s, m, l, alpha, c, nv8);
  pv_sub<D>(acc, cur, lds + ((u >> 1) % C::kStages) * C::kStageBytes + C::kTileBytes + (u & 1) * 32 * C::kRowBytes,
            voff);
  sub_exp<kMasked>(s, m, l, nxt, c, nv8);
  const unsigned flag = __builtin_amdgcn_readfirstlane(rescale ? 1u : 0u);
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
    scale_agpr_if(acc[db][0], alpha[0], flag);
    scale_agpr_if(acc[db][1], alpha[1], flag);
  }
}

template <int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
fa_fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
              __bf16* __restrict__ o, float* __restrict__ lse, int N, int tiles_per_head, int total_tiles,
              float c /* scale * log2(e) */) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];
  LDS_AS char* lds = (LDS_AS char*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;  // which half of the wave
  const int logical = remap_xcd(blockIdx.x, total_tiles);
  const int bh = logical / tiles_per_head;
  const int qtile = logical - bh * tiles_per_head;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const char* gk = (const char*)(k + head_off);
  const char* gv = (const char*)(v + head_off);
  const int T = (N + C::kBC - 1) / C::kBC;  // K/V tiles in LDS
  const int U = (N + 31) / 32;              // 32-key sub-tiles processed by the pipeline
  const int q0 = qtile * C::kBR + wave * C::kRowsPerWave;

  // Start streaming K/V tile 0 while Q is loaded.
  issue_tile<D>(gk, gv, 0, N, lds, wave, lane);

  // Q^T operand fragments: lane holds query q0 + qb*32 + lane%32, d = ks*16 + g*8 .. +8.
  bf16x8_t qf[2][C::kKS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 32 + (lane & 31);
    const bf16x8_t* src = (const bf16x8_t*)(q + head_off + (size_t)min(row, N - 1) * D + g * 8);
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      bf16x8_t x = src[ks * 2];
      if (row >= N) x = bf16x8_t{};
      qf[qb][ks] = x;
    }
  }

  // Per-lane LDS byte offsets of the operand reads (sub-tile base added later; the
  // swizzle depends on row bits 0-3 only, so 16-row-aligned bases keep it).
  int koff[C::kKS];
  {
    const int r0 = pi_row(lane & 31);
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) koff[ks] = chunk_offset<D>(r0, ks * 2 + g);
  }
  int voff[C::kDB][2];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 8 * g + 4 * r + ((lane & 15) >> 2);
      const int dcol = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db][r] = chunk_offset<D>(row, dcol >> 3) + 2 * (dcol & 7);
    }
  }

  float m[2] = {-__builtin_inff(), -__builtin_inff()};
  float l[2] = {0.0f, 0.0f};
  f32x16_t acc[C::kDB][2];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) acc[db][0] = acc[db][1] = f32x16_t{};

  wait_vmem();
  __syncthreads();
  if (T > 1) issue_tile<D>(gk, gv, 1, N, lds + C::kStageBytes, wave, lane);

  // Software pipeline over 32-key sub-tiles (see pipeline_step).
  const int nvalid_last = N - (U - 1) * 32;  // 1..32 keys in the last sub-tile
  const bool ragged = nvalid_last < 32;
  const int nv8 = nvalid_last - 8 * g;
  f32x16_t s[2];
  bf16x8_t pa[2][2], pb[2][2];
  {
    float alpha[2];
    qk_sub<D>(s, qf, lds, koff);
    if (U == 1 && ragged) {
      sub_max<true>(s, m, l, alpha, c, nv8);
      sub_exp<true>(s, m, l, pa, c, nv8);
    } else {
      sub_max<false>(s, m, l, alpha, c, nv8);
      sub_exp<false>(s, m, l, pa, c, nv8);
    }
  }
  int u = 0;
  for (; u + 2 < U; ++u) {
    pipeline_step<D, false>(u, T, N, gk, gv, lds, wave, lane, s, qf, koff, voff, m, l, acc, pa, pb, c, nv8);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      pa[qb][0] = pb[qb][0];
      pa[qb][1] = pb[qb][1];
    }
  }
  if (u + 1 < U) {  // u == U-2: the next sub-tile is the last one
    if (ragged) {
      pipeline_step<D, true>(u, T, N, gk, gv, lds, wave, lane, s, qf, koff, voff, m, l, acc, pa, pb, c, nv8);
    } else {
      pipeline_step<D, false>(u, T, N, gk, gv, lds, wave, lane, s, qf, koff, voff, m, l, acc, pa, pb, c, nv8);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      pa[qb][0] = pb[qb][0];
      pa[qb][1] = pb[qb][1];
    }
    ++u;
  }
  // Last sub-tile: PV only.
  pv_sub<D>(acc, pa, lds + ((u >> 1) % C::kStages) * C::kStageBytes + C::kTileBytes + (u & 1) * 32 * C::kRowBytes,
            voff);

  // Epilogue: O = acc / l (bf16, nearest-even), LSE = ln2 * (m + log2 l).
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lsum = pair_sum(l[qb]);
    const float inv = 1.0f / lsum;
    const int row = q0 + qb * 32 + (lane & 31);
    if (row < N) {
      __bf16* dst = o + head_off + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bf16x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][qb][i4 * 4 + e] * inv);
          *(bf16x4_t*)(dst + db * 32 + 8 * i4 + 4 * g) = w;
        }
      }
      if (g == 0) lse[(size_t)bh * N + row] = kLn2 * (m[qb] + log2f(lsum));
    }
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
                 float scale, const Blocks& blk, void* stream) {
  (void)blk;
  const int tiles = (N + 255) / 256;
  const long long total = (long long)B * H * tiles;
  const float c = scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  if (d == 128) {
    hipLaunchKernelGGL(fa_fwd_kernel<128>, dim3((unsigned)total), dim3(256), 0, s, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, N, tiles, (int)total, c);
  } else {
    hipLaunchKernelGGL(fa_fwd_kernel<64>, dim3((unsigned)total), dim3(256), 0, s, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, N, tiles, (int)total, c);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
