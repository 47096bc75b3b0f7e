// Attention backward on gfx950: dQ, dK, dV of O = softmax(scale * Q K^T) V for an
// upstream dO, from Q, K, V and the forward's O and LSE.
//
// The pages keep only O and the per-row LSE from the forward and recompute P in
// the backward instead of storing it ("01 · 注意力为什么是 IO 瓶颈", section 6), so
// no N x N matrix is stored here either. Per (b, h), with P = exp(S - LSE):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q
// where D_i = dO_i . O_i equals sum_j P_ij dP_ij (the softmax Jacobian's row term).
//
// Three kernels:
//   bwd_pre   D (fp32) and LSE in log2 units, per query row, into the workspace;
//   bwd_dq    one workgroup per 128 query rows: streams 32-key K/V tiles through
//             LDS, recomputes S^T = K Q^T and dP^T = V dO^T, and accumulates
//             dQ^T += K^T dS^T (the forward kernel's orientation: each lane owns one
//             query column, K^T comes from LDS through transposing reads);
//   bwd_dkdv  one workgroup per 128 keys, K and V held in registers: streams
//             32-row Q/dO tiles through LDS, recomputes S = Q K^T and dP = dO V^T, and
//             accumulates dV^T += dO^T P and dK^T += Q^T dS (each lane owns one key
//             column; dO^T and Q^T come from LDS through transposing reads). At
//             d = 128 (bwd_dkdv_pair) the work of 32 keys is split over two waves
//             that share a SIMD, one for S, P and dV, the other for dP, dS and dK.
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS enter
// them as bf16 (nearest-even). The row order inside a 32-row block of the operand
// read from LDS as rows is permuted (bits 2 and 3 swapped), which makes the
// accumulator layout of S (or S^T) equal to the operand layout of the next
// product's transposing read, as in the forward kernel.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// LDS tile layout: rows of D bf16 as D/8 16-byte chunks, the chunk index XORed
// with a function of the row's low 4 bits, so that 16-row reads of one chunk and
// the 4-row transposing reads both spread over the LDS banks (the same layout as
// the forward kernel's K/V stages; 16-row-aligned offsets keep it).
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
// Operand row rho of a 32-row block reads tile row pi(rho): bits 2 and 3 swapped.
__device__ __forceinline__ int pi_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Tile row held by accumulator register i of a lane in half g (g = lane / 32) after
// a product whose rows were read through pi_row: pi(8*(i/4) + 4g + i%4).
__device__ __forceinline__ constexpr int acc_row(int i, int g) {
  return 16 * (i >> 3) + 8 * g + 4 * ((i >> 2) & 1) + (i & 3);
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// MFMAs with pinned register classes for the dK/dV kernel, whose two d x 32
// accumulators stay in AGPRs for the whole kernel and whose K and V operands sit in
// AGPRs as B sources. The compiler does not see these as MFMAs, so the kernel keeps
// the wait states itself: VALU code reads S and dP only after an s_nop pin that
// follows the products writing them, the packed P and dS get an s_nop before the
// products that read them, and the accumulators get sync_acc before VALU reads.
__device__ __forceinline__ void mfma_sv(f32x16_t& d, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_sv0(f32x16_t& d, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16_t& d, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Wait states between the last MFMA writing a VGPR result and VALU reads of it.
__device__ __forceinline__ void sync_sv(f32x16_t& a, f32x16_t& b) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+v"(a), "+v"(b));
}
// ... and between the last MFMA writing an AGPR accumulator and VALU reads of it.
__device__ __forceinline__ void sync_acc(f32x16_t& a, f32x16_t& b) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+a"(a), "+a"(b));
}

// Eight accumulator values -> one bf16x8 operand (nearest-even), element order kept.
__device__ __forceinline__ bf16x8_t pack8(const float* x) {
  const bf16x2_t p0 = __builtin_convertvector((f32x2_t){x[0], x[1]}, bf16x2_t);
  const bf16x2_t p1 = __builtin_convertvector((f32x2_t){x[2], x[3]}, bf16x2_t);
  const bf16x2_t p2 = __builtin_convertvector((f32x2_t){x[4], x[5]}, bf16x2_t);
  const bf16x2_t p3 = __builtin_convertvector((f32x2_t){x[6], x[7]}, bf16x2_t);
  return __builtin_bit_cast(bf16x8_t, (u32x4_t){__builtin_bit_cast(unsigned, p0), __builtin_bit_cast(unsigned, p1),
                                                  __builtin_bit_cast(unsigned, p2), __builtin_bit_cast(unsigned, p3)});
}

// Workgroup id -> logical tile id such that each XCD (ids w with w % 8 == x) gets
// a contiguous range: a head's tiles share one L2.
__device__ __forceinline__ int remap_xcd(int w, int total) {
  const int xcd = w & 7, idx = w >> 3;
  const int base = total >> 3, rem = total & 7;
  return xcd < rem ? xcd * (base + 1) + idx : rem * (base + 1) + (xcd - rem) * base + idx;
}

// Buffer resource over rows [row0, row0 + rows) of an array of `row_bytes`-wide rows
// that has N rows: only the part inside N is mapped, so loads past it return zeros
// without touching memory (the ragged last tile, and tiles past the end, need no
// clamping). Word 3 selects raw 32-bit data (no swizzle, no index stride).
constexpr unsigned kRawBufferWord3 = 0x00020000u;
__device__ __forceinline__ u32x4_t rows_rsrc(const void* base, int row0, int rows, int N, int row_bytes) {
  const int valid = min(max(N - row0, 0), rows);
  const uint64_t a = (uint64_t)(uintptr_t)base + (uint64_t)(int64_t)row0 * (uint64_t)row_bytes;
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane((unsigned)(valid * row_bytes));
  r[3] = kRawBufferWord3;
  return r;
}

// Direct global->LDS loads (buffer_load ... lds): lane l's 16 (or 4) bytes at byte
// offset voff of the resource land at LDS address lds_addr + 16*l (or 4*l). Issued
// through asm so that the compiler does not put a vmcnt(0) wait in front of every
// LDS read (it cannot tell that the destination stage is not the one being read);
// the kernel waits for these loads itself (tile_barrier). M0 carries the LDS
// address, with one wait state between its write and the load. The compiler warns
// that M0 is reserved and its clobber not honoured: no other code in these kernels
// uses M0, and each of these asm blocks sets it before its load.
__device__ __forceinline__ void dma16(u32x4_t rsrc, unsigned voff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(u32x4_t rsrc, unsigned voff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Wait until at most kOutstanding of this wave's vector-memory loads are in flight
// (they complete in issue order), then the workgroup barrier: after it every wave's
// share of the tiles older than those is in LDS. The memory clobbers keep the
// compiler from moving LDS accesses across it.
template <int kOutstanding>
__device__ __forceinline__ void tile_barrier() {
  static_assert(kOutstanding >= 0 && kOutstanding <= 63, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOutstanding) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// ---- kernel 1: D_i = dO_i . O_i and LSE_i * log2(e) ----
// D/8 lanes per row (8 elements each), 64*8/D rows per wave.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dO,
                                                      const float* __restrict__ lse, float* __restrict__ dvec,
                                                      float* __restrict__ lse2, long long rows) {
  constexpr int kLanes = D / 8, kRowsPerWave = 64 / kLanes;
  const int lane = threadIdx.x & 63, t = lane % kLanes;
  const long long row = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * kRowsPerWave + lane / kLanes;
  float s = 0.0f;
  if (row < rows) {
    const u32x4_t a = *(const u32x4_t*)(o + row * D + 8 * t);
    const u32x4_t b = *(const u32x4_t*)(dO + row * D + 8 * t);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned aj = a[j], bj = b[j];
      s = __builtin_fmaf(__builtin_bit_cast(float, aj << 16), __builtin_bit_cast(float, bj << 16), s);
      s = __builtin_fmaf(__builtin_bit_cast(float, aj & 0xFFFF0000u), __builtin_bit_cast(float, bj & 0xFFFF0000u), s);
    }
  }
  s += dpp<0xB1>(s);   // quad_perm [1,0,3,2]
  s += dpp<0x4E>(s);   // quad_perm [2,3,0,1]
  s += dpp<0x141>(s);  // row_half_mirror
  if constexpr (D == 128) s += dpp<0x140>(s);  // row_mirror
  if (row < rows && t == 0) {
    dvec[row] = s;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ---- kernel 2: dQ ----
// Two waves per SIMD (232 VGPRs at d = 128): one wave's softmax and LDS reads
// overlap the other's products.
template <int D>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                     const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
                                                     const float* __restrict__ dvec, const float* __restrict__ lse2,
                                                     __bf16* __restrict__ dq, int N, int tiles_per_head,
                                                     int total_tiles, float c, float scale) {
  constexpr int KS = D / 16, DB = D / 32, kTile = 32 * D * 2;
  // Ring of 32-key K/V tiles: each stage holds the K tile, then the V tile.
  constexpr int kStages = 4, kStage = 2 * kTile;
  constexpr int kChunks = D / 8;
  constexpr int kLoads = kTile / 1024 / 4;  // 16-byte loads per wave per K (or V) tile
  constexpr int kPerTile = 2 * kLoads;      // this wave's loads per K/V tile
  static_assert(kLoads >= 1 && kTile % 4096 == 0, "tile loads must split evenly over the 4 waves");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];
  const unsigned lds = (unsigned)(uintptr_t)(LDS_AS char*)smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  const int logical = remap_xcd(blockIdx.x, total_tiles);
  const int bh = logical / tiles_per_head, qt = logical % tiles_per_head;
  const size_t head = (size_t)bh * N * D;
  const int qrow = qt * 128 + wave * 32 + (lane & 31);

  bf16x8_t qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = bf16x8_t{};
    df[ks] = bf16x8_t{};
    if (qrow < N) {
      qf[ks] = *(const bf16x8_t*)(q + head + (size_t)qrow * D + ks * 16 + g * 8);
      df[ks] = *(const bf16x8_t*)(dO + head + (size_t)qrow * D + ks * 16 + g * 8);
    }
  }
  float lq = qrow < N ? lse2[(size_t)bh * N + qrow] : __builtin_inff();  // padded rows: P = 0
  float dd = qrow < N ? dvec[(size_t)bh * N + qrow] : 0.0f;
  // Consumed here, so the compiler waits for these loads once, in the prologue. Left
  // to the loop, it would wait for them there with vmcnt(0) every step, which also
  // waits for the K/V tile loads in flight (it does not count the asm loads), and
  // the tiles would no longer load ahead.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]), "+v"(df[ks]));
  asm volatile("" : "+v"(lq), "+v"(dd));
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  const int T = (N + 31) / 32;
  // K and V rows go straight from global memory into a stage (buffer_load ... lds,
  // 16 bytes per lane, in the swizzled layout that read_row and read_tr expect):
  // lane l's load i is slot p = (wave * kLoads + i) * 64 + l of the tile, row
  // p / kChunks, logical chunk (p % kChunks) ^ swz. Keys past N read as zeros, and
  // their P is set to 0 below.
  unsigned gofs[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = (wave * kLoads + i) * 64 + lane, row = p / kChunks;
    gofs[i] = (unsigned)(row * D * 2 + (((p % kChunks) ^ swz<D>(row)) << 4));
  }
  const char* kh = (const char*)(k + head);
  const char* vh = (const char*)(v + head);
  auto issue = [&](int u, unsigned st) {
    const u32x4_t rk = rows_rsrc(kh, u * 32, 32, N, D * 2);
    const u32x4_t rv = rows_rsrc(vh, u * 32, 32, N, D * 2);
    const unsigned dst = __builtin_amdgcn_readfirstlane(st + (unsigned)(wave * kLoads * 1024));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dma16(rk, gofs[i], dst + i * 1024);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dma16(rv, gofs[i], dst + kTile + i * 1024);
  };
  // Per-lane LDS addresses of the operand reads for a stage at offset 0 (as in the
  // dK/dV kernel): the loop is unrolled over the four ring stages, so each stage
  // offset rides in the ds_read immediate.
  unsigned rofs[KS], tofs[DB][2];
  {
    const int rr = pi_row(lane & 31), trow = 8 * g + ((lane & 15) >> 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      rofs[ks] = lds + (unsigned)chunk_offset<D>(rr, 2 * ks + g);
      asm volatile("" : "+v"(rofs[ks]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      tofs[db][0] = lds + (unsigned)(chunk_offset<D>(trow, col >> 3) + 2 * (col & 7));
      tofs[db][1] = lds + (unsigned)(chunk_offset<D>(trow + 4, col >> 3) + 2 * (col & 7));
      asm volatile("" : "+v"(tofs[db][0]), "+v"(tofs[db][1]));
    }
  }
  static_assert((kStages - 1) * kStage + kTile + 16 * 2 * D < 65536, "stage offsets must fit the ds_read immediate");
  auto rd_row = [&](unsigned off, int ks) -> bf16x8_t {
    return *(const LDS_AS bf16x8_t*)(uintptr_t)(rofs[ks] + off);
  };
  auto rd_tr = [&](unsigned off, int db) -> bf16x8_t {
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(uintptr_t)(tofs[db][0] + off));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(uintptr_t)(tofs[db][1] + off));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4,
                                   5, 6, 7);
  };
  // Tile t+3's loads go out during step t into the stage tile t-1 used (its reads
  // were consumed by step t-1's products, before the barrier ending that step); the
  // barrier ending step t+2 waits for them, so each tile has three steps to land.
  // Step t uses stage t % 4 (J below). Only the ragged last tile (kMasked) sets the
  // P of keys >= N to zero; in every other tile all 32 keys are inside N. (A padded
  // key's K row is zero, so its dS would add nothing to dQ anyway, but its P =
  // exp2(-LSE2) could overflow for rows whose LSE is very negative, and 0 * inf is
  // not 0.)
  auto step = [&](auto j_tag, auto masked_tag, int t) {
    constexpr int J = decltype(j_tag)::value;
    constexpr bool kMasked = decltype(masked_tag)::value;
    constexpr unsigned KT = J * kStage, VT = KT + kTile;
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
    // Two waves share each SIMD. A wave raises its issue priority while it issues
    // its S and dP products (and a later tile's loads), so that the matrix core is
    // fed by the wave in that phase while the other runs its softmax on the VALU
    // (at B=1 H=32 N=8192 d=128: kernel cycles -11%, matrix cores 0.69 -> 0.78 busy).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma(rd_row(KT, ks), qf[ks], s);
      dp = mfma(rd_row(VT, ks), df[ks], dp);
    }
    // Issued after the S/dP reads, so those start right after the barrier (the
    // loads' asm is a compiler memory fence).
    issue(t + kStages - 1, lds + (unsigned)(((J + kStages - 1) % kStages) * kStage));
    __builtin_amdgcn_s_setprio(0);
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -lq));
      if constexpr (kMasked) {
        if (t * 32 + acc_row(i, g) >= N) p = 0.0f;
      }
      ds[i] = p * (dp[i] - dd);
    }
    const bf16x8_t b0 = pack8(ds), b1 = pack8(ds + 8);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma(rd_tr(KT, db), b0, acc[db]);
      acc[db] = mfma(rd_tr(KT + 16 * 2 * D, db), b1, acc[db]);
    }
    // Tile t+1 has landed; tiles t+2 and t+3 may stay in flight.
    tile_barrier<2 * kPerTile>();
  };
#pragma unroll
  for (int u = 0; u < kStages - 1; ++u) issue(u, lds + (unsigned)(u * kStage));
  tile_barrier<2 * kPerTile>();  // tile 0 landed; tiles 1 and 2 may stay in flight
  static_assert(kStages == 4, "the unrolled loop below covers a ring of four stages");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using Full = std::false_type;
  using Ragged = std::true_type;
  const int TF = N / 32;  // tiles with all 32 keys inside N
  int t = 0;
  for (; t + kStages <= TF; t += kStages) {
    step(I0{}, Full{}, t);
    step(I1{}, Full{}, t + 1);
    step(I2{}, Full{}, t + 2);
    step(I3{}, Full{}, t + 3);
  }
  if (t < TF) step(I0{}, Full{}, t);
  if (t + 1 < TF) step(I1{}, Full{}, t + 1);
  if (t + 2 < TF) step(I2{}, Full{}, t + 2);
  if (TF < T) {  // the ragged last tile, in stage TF % 4
    switch (TF & 3) {
      case 0: step(I0{}, Ragged{}, TF); break;
      case 1: step(I1{}, Ragged{}, TF); break;
      case 2: step(I2{}, Ragged{}, TF); break;
      default: step(I3{}, Ragged{}, TF); break;
    }
  }
  // Loads issued past the last tile (zero fills) must land before the workgroup's
  // LDS can be handed to another workgroup.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // Lane holds dQ^T rows (columns of dQ) db*32 + 8*(i/4) + 4g + i%4 of query qrow.
  if (qrow < N) {
    __bf16* out = dq + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x2_t a = {acc[db][4 * i4] * scale, acc[db][4 * i4 + 1] * scale};
        const f32x2_t b = {acc[db][4 * i4 + 2] * scale, acc[db][4 * i4 + 3] * scale};
        const u32x2_t w = {__builtin_bit_cast(unsigned, __builtin_convertvector(a, bf16x2_t)),
                           __builtin_bit_cast(unsigned, __builtin_convertvector(b, bf16x2_t))};
        *(u32x2_t*)(out + db * 32 + 8 * i4 + 4 * g) = w;
      }
    }
  }
}

// ---- kernel 3: dK and dV, one wave per 32 keys (run at d = 64) ----
// Two waves per SIMD at d = 64. At d = 128 the two d x 32 accumulators, K and V
// (192 AGPRs) and about 160 VGPRs would leave room for one, so d = 128 runs the
// two-wave kernel below instead.
template <int D>
__global__ void __launch_bounds__(256, D == 64 ? 2 : 1) bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                       const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
                                                       const float* __restrict__ dvec, const float* __restrict__ lse2,
                                                       __bf16* __restrict__ dk, __bf16* __restrict__ dv, int N,
                                                       int tiles_per_head, int total_tiles, float c, float scale) {
  constexpr int KS = D / 16, DB = D / 32, kTile = 32 * D * 2;
  // Ring of Q/dO tiles of 32 rows: each stage holds the Q tile, the dO tile and a
  // 1 KB vector area (LSE2 of the tile's rows at +0, D at +256; +512 and +768 take
  // the zero fills of the vector loads that waves 2 and 3 issue so that every wave
  // issues the same number of loads per tile).
  constexpr int kStages = 4, kVec = 1024;
  constexpr int kStage = 2 * kTile + kVec;
  constexpr int kChunks = D / 8;
  constexpr int kLoads = kTile / 1024 / 4;  // 16-byte loads per wave per Q (or dO) tile
  constexpr int kPerTile = 2 * kLoads + 1;  // this wave's loads per tile, vector load included
  static_assert(kLoads >= 1 && kTile % 4096 == 0, "tile loads must split evenly over the 4 waves");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];
  const unsigned lds = (unsigned)(uintptr_t)(LDS_AS char*)smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  const int logical = remap_xcd(blockIdx.x, total_tiles);
  const int bh = logical / tiles_per_head, kt0 = logical % tiles_per_head;
  const size_t head = (size_t)bh * N * D;
  const size_t rowvec = (size_t)bh * N;
  const int krow = kt0 * 128 + wave * 32 + (lane & 31);

  bf16x8_t kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = bf16x8_t{};
    vf[ks] = bf16x8_t{};
    if (krow < N) {
      kf[ks] = *(const bf16x8_t*)(k + head + (size_t)krow * D + ks * 16 + g * 8);
      vf[ks] = *(const bf16x8_t*)(v + head + (size_t)krow * D + ks * 16 + g * 8);
    }
  }
  // K and V into AGPRs, with the wait states before the first MFMA that reads them.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("s_nop 1" : "+a"(kf[ks]), "+a"(vf[ks]));
  asm volatile("s_nop 7" ::: "memory");
  f32x16_t adk[DB], adv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    adk[db] = f32x16_t{};
    adv[db] = f32x16_t{};
  }

  const int T = (N + 31) / 32;
  // Loads: tile u's Q and dO rows go straight from global memory into a stage
  // (buffer_load ... lds, 16 bytes per lane, in the swizzled layout that read_row and
  // read_tr expect), and so do its 32 LSE2 and D values (4 bytes per lane). Lane l's
  // 16 bytes of load i form slot p = (wave * kLoads + i) * 64 + l of the tile: row
  // p / kChunks, physical chunk p % kChunks, i.e. logical chunk (p % kChunks) ^ swz.
  unsigned gofs[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = (wave * kLoads + i) * 64 + lane, row = p / kChunks;
    gofs[i] = (unsigned)(row * D * 2 + (((p % kChunks) ^ swz<D>(row)) << 4));
  }
  const char* qh = (const char*)(q + head);
  const char* dh = (const char*)(dO + head);
  // part 0: Q rows, 1: dO rows, 2: the vector (wave 0 LSE2, wave 1 D, waves 2-3 an
  // empty resource). Rows past N, and tiles past the end, read as zeros: their Q and
  // dO rows are zero, so S = 0 and P = exp2(0 - 0) = 1 there, while dP = D = 0 gives
  // dS = 0 and the zero dO row adds nothing to dV.
  auto issue = [&](int part, int u, unsigned st) {
    if (part < 2) {
      const u32x4_t r = rows_rsrc(part == 0 ? qh : dh, u * 32, 32, N, D * 2);
      const unsigned dst = __builtin_amdgcn_readfirstlane(st + (unsigned)(part * kTile + wave * kLoads * 1024));
#pragma unroll
      for (int i = 0; i < kLoads; ++i) dma16(r, gofs[i], dst + i * 1024);
    } else {
      const float* src = (wave == 0 ? lse2 : dvec) + rowvec;
      const u32x4_t r = rows_rsrc(src, u * 32, 32, wave < 2 ? N : 0, 4);
      dma4(r, (unsigned)lane * 4u, __builtin_amdgcn_readfirstlane(st + (unsigned)(2 * kTile + wave * 256)));
    }
  };
  // Per-lane LDS addresses of the operand reads for a stage at offset 0:
  //  * row reads: for k-step ks, lane l receives chunk 2*ks + g of tile row
  //    pi(l % 32), the row operand of a product that contracts over d;
  //  * transposing reads (ds_read_b64_tr_b16): for column block db, lane l receives
  //    the 8 values of column db*32 + l%32 in rows 8g .. 8g+7, as two reads of four
  //    rows each: the A operand of a product that contracts over those rows. Rows
  //    16-31 are 16 rows further, the swizzle depending on row bits 0-3 only.
  // The loop below is unrolled over the four stages
  // of the ring, so every stage offset is a constant and rides in the ds_read
  // immediate (at most 3 * kStage + kTile + 16 rows < 64 KiB): no address
  // arithmetic per read. The empty asm keeps the compiler from recomputing them.
  unsigned rofs[KS], tofs[DB][2];
  {
    const int rr = pi_row(lane & 31), trow = 8 * g + ((lane & 15) >> 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      rofs[ks] = lds + (unsigned)chunk_offset<D>(rr, 2 * ks + g);
      asm volatile("" : "+v"(rofs[ks]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      tofs[db][0] = lds + (unsigned)(chunk_offset<D>(trow, col >> 3) + 2 * (col & 7));
      tofs[db][1] = lds + (unsigned)(chunk_offset<D>(trow + 4, col >> 3) + 2 * (col & 7));
      asm volatile("" : "+v"(tofs[db][0]), "+v"(tofs[db][1]));
    }
  }
  static_assert((kStages - 1) * kStage + kTile + 16 * 2 * D < 65536, "stage offsets must fit the ds_read immediate");
  auto rd_row = [&](unsigned off, int ks) -> bf16x8_t {
    return *(const LDS_AS bf16x8_t*)(uintptr_t)(rofs[ks] + off);
  };
  auto rd_tr = [&](unsigned off, int db) -> bf16x8_t {
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(uintptr_t)(tofs[db][0] + off));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(uintptr_t)(tofs[db][1] + off));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4,
                                   5, 6, 7);
  };
  // S and dP of a tile: KS products each, in ks order. The row operands are read one
  // window ahead: loads do not move across the asm MFMAs, so reading them right
  // before their product would expose the LDS latency.
  auto sdp_step = [&](int ks, const bf16x8_t& aq, const bf16x8_t& ad, f32x16_t& s, f32x16_t& dp) {
    if (ks == 0) {
      mfma_sv0(s, aq, kf[ks]);
      mfma_sv0(dp, ad, vf[ks]);
    } else {
      mfma_sv(s, aq, kf[ks]);
      mfma_sv(dp, ad, vf[ks]);
    }
  };
  // Pipeline: while tile t's softmax runs on the VALU, the matrix cores compute S
  // and dP of tile t+1, and tiles t+2 and t+3 are in flight from memory: tile t+3's
  // loads go out during step t into the stage that tile t-1 used (its last reads
  // were consumed by step t-1's products, before the barrier ending that step), and
  // the barrier ending step t+1 waits for them. The softmax is cut into four parts,
  // one per group of S/dP products, and within a part each product slot carries the
  // VALU work of one or two elements, so that work runs beside the MFMAs. Each part
  // is pinned to its place (inputs at its start, outputs at its end). Tiles past
  // the end are zero rows, so every step runs the same code. Step t uses stage
  // t % 4 (J below); S and dP alternate between two register sets, so no copy is
  // needed between steps.
  constexpr int kPer = KS / 4;
  auto step = [&](auto j_tag, int t, f32x16_t& s, f32x16_t& dp, f32x16_t& s2, f32x16_t& dp2) {
    constexpr int J = decltype(j_tag)::value;
    constexpr unsigned CUR = J * kStage, NXT = ((J + 1) % kStages) * kStage;
    constexpr unsigned FUT = ((J + kStages - 1) % kStages) * kStage;
    const LDS_AS float* l2v = (const LDS_AS float*)(uintptr_t)(lds + CUR + 2 * kTile);
    const LDS_AS float* dvv = l2v + 64;
    float p[16], ds[16];
    // LSE2 and D of the four softmax parts' rows, read at the step start.
    f32x4_t l4s[4], d4s[4];
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      const int r = acc_row(4 * part, g);
      l4s[part] = *(const LDS_AS f32x4_t*)(l2v + r);
      d4s[part] = *(const LDS_AS f32x4_t*)(dvv + r);
    }
    bf16x8_t rq[KS], rd[KS];  // row operands of tile t+1; only a window is live at once
#pragma unroll
    for (int ks = 0; ks < kPer; ++ks) {
      rq[ks] = rd_row(NXT, ks);
      rd[ks] = rd_row(NXT + kTile, ks);
    }
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      if (part < 3) issue(part, t + kStages - 1, lds + FUT);
      if (part + 1 < 4) {
#pragma unroll
        for (int ks = (part + 1) * kPer; ks < (part + 2) * kPer; ++ks) {
          rq[ks] = rd_row(NXT, ks);
          rd[ks] = rd_row(NXT + kTile, ks);
        }
      }
      // Softmax of rows acc_row(4*part, g) .. +3 of tile t, spread over this part's
      // 2*kPer product slots: each slot issues one MFMA, then the fma, exp2, sub and
      // mul of its elements, which run on the VALU while the MFMA does. A fence
      // closes each slot so the compiler cannot gather the VALU work in one place.
      float sx[4], dx[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sx[j] = s[4 * part + j];
        dx[j] = dp[4 * part + j];
      }
      asm volatile("" : "+v"(sx[0]), "+v"(sx[1]), "+v"(sx[2]), "+v"(sx[3]), "+v"(dx[0]), "+v"(dx[1]), "+v"(dx[2]),
                   "+v"(dx[3]));
      constexpr int kSlots = 2 * kPer;
#pragma unroll
      for (int m = 0; m < kSlots; ++m) {
        const int ks = part * kPer + m / 2;
        if (m % 2 == 0) {
          if (ks == 0) mfma_sv0(s2, rq[ks], kf[ks]);
          else mfma_sv(s2, rq[ks], kf[ks]);
        } else {
          if (ks == 0) mfma_sv0(dp2, rd[ks], vf[ks]);
          else mfma_sv(dp2, rd[ks], vf[ks]);
        }
#pragma unroll
        for (int j = m * 4 / kSlots; j < (m + 1) * 4 / kSlots; ++j) {
          const int i = 4 * part + j;
          p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[j], c, -l4s[part][j]));
          ds[i] = p[i] * (dx[j] - d4s[part][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      asm volatile("" : "+v"(p[4 * part]), "+v"(p[4 * part + 1]), "+v"(p[4 * part + 2]), "+v"(p[4 * part + 3]),
                   "+v"(ds[4 * part]), "+v"(ds[4 * part + 1]), "+v"(ds[4 * part + 2]), "+v"(ds[4 * part + 3]));
    }
    // Transposed operands of the accumulator products (dO^T for dV, Q^T for dK, rows
    // 0-15 and 16-31 of the tile), read one column block ahead.
    bf16x8_t tr[DB][4];
    auto read_block = [&](int db) {
      tr[db][0] = rd_tr(CUR + kTile, db);
      tr[db][1] = rd_tr(CUR + kTile + 16 * 2 * D, db);
      tr[db][2] = rd_tr(CUR, db);
      tr[db][3] = rd_tr(CUR + 16 * 2 * D, db);
    };
    read_block(0);
    bf16x8_t p0 = pack8(p), p1 = pack8(p + 8), s0 = pack8(ds), s1 = pack8(ds + 8);
    // Two wait states between the VALU writes of the operands and the MFMAs reading them.
    asm volatile("s_nop 1" : "+v"(p0), "+v"(p1), "+v"(s0), "+v"(s1));
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db + 1 < DB) read_block(db + 1);
      mfma_acc(adv[db], tr[db][0], p0);
      mfma_acc(adv[db], tr[db][1], p1);
      mfma_acc(adk[db], tr[db][2], s0);
      mfma_acc(adk[db], tr[db][3], s1);
    }
    // Tile t+2 (read from step t+1 on) has landed; tile t+3 may stay in flight.
    tile_barrier<kPerTile>();
    // The products of S2 and dP2 were issued before the 4*DB accumulator products,
    // which issue in order behind them on the same matrix core, so their results are
    // written long before the next step's VALU reads them; the s_nop adds the two
    // wait states of a VALU read after an MFMA issue, and the pin keeps those reads
    // after this point.
    asm volatile("s_nop 1" : "+v"(s2), "+v"(dp2));
  };
#pragma unroll
  for (int u = 0; u < kStages - 1; ++u) {
    const unsigned st = lds + (unsigned)(u * kStage);
    issue(0, u, st);
    issue(1, u, st);
    issue(2, u, st);
  }
  tile_barrier<kPerTile>();  // tiles 0 and 1 landed; tile 2 may stay in flight
  f32x16_t sA, dpA, sB, dpB;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) sdp_step(ks, rd_row(0, ks), rd_row(kTile, ks), sA, dpA);
  sync_sv(sA, dpA);
  static_assert(kStages == 4, "the unrolled loop below covers a ring of four stages");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  int t = 0;
  for (; t + kStages <= T; t += kStages) {
    step(I0{}, t, sA, dpA, sB, dpB);
    step(I1{}, t + 1, sB, dpB, sA, dpA);
    step(I2{}, t + 2, sA, dpA, sB, dpB);
    step(I3{}, t + 3, sB, dpB, sA, dpA);
  }
  if (t < T) step(I0{}, t, sA, dpA, sB, dpB);
  if (t + 1 < T) step(I1{}, t + 1, sB, dpB, sA, dpA);
  if (t + 2 < T) step(I2{}, t + 2, sA, dpA, sB, dpB);
  // Loads issued past the last tile (zero fills) must land before the workgroup's
  // LDS can be handed to another workgroup.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int db = 0; db < DB; ++db) sync_acc(adk[db], adv[db]);
  if (krow < N) {
    __bf16* ok = dk + head + (size_t)krow * D;
    __bf16* ov = dv + head + (size_t)krow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = db * 32 + 8 * i4 + 4 * g;
        const f32x2_t ka = {adk[db][4 * i4] * scale, adk[db][4 * i4 + 1] * scale};
        const f32x2_t kb = {adk[db][4 * i4 + 2] * scale, adk[db][4 * i4 + 3] * scale};
        const f32x2_t va = {adv[db][4 * i4], adv[db][4 * i4 + 1]};
        const f32x2_t vb = {adv[db][4 * i4 + 2], adv[db][4 * i4 + 3]};
        *(u32x2_t*)(ok + col) = u32x2_t{__builtin_bit_cast(unsigned, __builtin_convertvector(ka, bf16x2_t)),
                                        __builtin_bit_cast(unsigned, __builtin_convertvector(kb, bf16x2_t))};
        *(u32x2_t*)(ov + col) = u32x2_t{__builtin_bit_cast(unsigned, __builtin_convertvector(va, bf16x2_t)),
                                        __builtin_bit_cast(unsigned, __builtin_convertvector(vb, bf16x2_t))};
      }
    }
  }
}

// ---- kernel 3, d = 128: dK and dV with two waves per SIMD ----
// Eight waves per workgroup of 128 keys, in pairs that share 32 keys. Waves 0-3
// (the P role) hold K and the dV^T accumulator: per 32-row tile they compute
// S = Q K^T and P = exp2(S c - LSE2), hand P (fp32) to their partner through LDS,
// and accumulate dV^T += dO^T P. Waves 4-7 (the dS role) hold V and the dK^T
// accumulator: they compute dP = dO V^T, take P from LDS, form dS = P o (dP - D)
// and accumulate dK^T += Q^T dS. Each role runs 16 of a tile's 32 products, and a
// SIMD holds one wave of each role (waves w and w + 4 of a workgroup share a SIMD),
// so while one wave waits on its products or on LDS the other issues. The P role works one tile ahead: in step s it takes tile
// s + 1 while its partner takes tile s, whose P it wrote in step s - 1. Every
// product, the P and dS values and the accumulation order are those of the
// one-wave kernel above, so the two give bitwise-equal gradients.
template <int D>
__global__ void __launch_bounds__(512, 1) bwd_dkdv_pair_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                             const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
                                                             const float* __restrict__ dvec, const float* __restrict__ lse2,
                                                             __bf16* __restrict__ dk, __bf16* __restrict__ dv, int N,
                                                             int tiles_per_head, int total_tiles, float c, float scale) {
  constexpr int KS = D / 16, DB = D / 32, kTile = 32 * D * 2;
  constexpr int kWaves = 8;
  // Ring of Q/dO tiles of 32 rows: each stage holds the Q tile, the dO tile and a
  // 1 KB vector area (LSE2 of the tile's rows at +0, D at +256; +512 takes the zero
  // fills of the vector loads that waves 2-7 issue so that every wave issues the
  // same number of loads per tile).
  constexpr int kStages = 4, kVec = 1024;
  constexpr int kStage = 2 * kTile + kVec;
  constexpr int kChunks = D / 8;
  constexpr int kLoads = kTile / 1024 / kWaves;  // 16-byte loads per wave per Q (or dO) tile
  constexpr int kPerTile = 2 * kLoads + 1;       // this wave's loads per tile, vector load included
  constexpr int kX = 32 * 32 * 4;                // one pair's P of one tile, fp32
  static_assert(kLoads >= 1 && kTile % (1024 * kWaves) == 0, "tile loads must split evenly over the 8 waves");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];
  __shared__ __attribute__((aligned(1024))) char xch[2 * 4 * kX];  // P hand-over, two tiles x four pairs
  const unsigned lds = (unsigned)(uintptr_t)(LDS_AS char*)smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  const int pair = wave & 3;
  const bool role_p = wave < 4;
  const int logical = remap_xcd(blockIdx.x, total_tiles);
  const int bh = logical / tiles_per_head, kt0 = logical % tiles_per_head;
  const size_t head = (size_t)bh * N * D;
  const size_t rowvec = (size_t)bh * N;
  const int krow = kt0 * 128 + pair * 32 + (lane & 31);

  // K (P role) or V (dS role) of the pair's 32 keys: the B operand of S or dP.
  const __bf16* kvsrc = role_p ? k : v;
  bf16x8_t kv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kv[ks] = bf16x8_t{};
    if (krow < N) kv[ks] = *(const bf16x8_t*)(kvsrc + head + (size_t)krow * D + ks * 16 + g * 8);
  }
  // Consumed here, so the compiler waits for these loads once, in the prologue,
  // rather than with a vmcnt(0) inside the loop, which would also wait for the
  // tile loads in flight (the compiler does not count the asm loads).
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(kv[ks]));
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  const int T = (N + 31) / 32;
  // Loads as in the one-wave kernel, over eight waves: lane l's 16 bytes of load i
  // form slot p = (wave * kLoads + i) * 64 + l of the tile.
  unsigned gofs[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = (wave * kLoads + i) * 64 + lane, row = p / kChunks;
    gofs[i] = (unsigned)(row * D * 2 + (((p % kChunks) ^ swz<D>(row)) << 4));
  }
  const char* qh = (const char*)(q + head);
  const char* dh = (const char*)(dO + head);
  const float* vsrc = (wave == 0 ? lse2 : dvec) + rowvec;
  const unsigned vdst = wave < 2 ? (unsigned)(2 * kTile + wave * 256) : (unsigned)(2 * kTile + 512);
  auto issue = [&](int u, unsigned st) {
    const u32x4_t rq = rows_rsrc(qh, u * 32, 32, N, D * 2);
    const u32x4_t rd = rows_rsrc(dh, u * 32, 32, N, D * 2);
    const unsigned dst = __builtin_amdgcn_readfirstlane(st + (unsigned)(wave * kLoads * 1024));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dma16(rq, gofs[i], dst + i * 1024);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dma16(rd, gofs[i], dst + kTile + i * 1024);
    const u32x4_t rv = rows_rsrc(vsrc, u * 32, 32, wave < 2 ? N : 0, 4);
    dma4(rv, (unsigned)lane * 4u, __builtin_amdgcn_readfirstlane(st + vdst));
  };
  // Per-lane LDS addresses of the operand reads for a stage at offset 0, as in the
  // one-wave kernel; the loop is unrolled over the four ring stages, so each stage
  // offset rides in the ds_read immediate.
  unsigned rofs[KS], tofs[DB][2];
  {
    const int rr = pi_row(lane & 31), trow = 8 * g + ((lane & 15) >> 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      rofs[ks] = lds + (unsigned)chunk_offset<D>(rr, 2 * ks + g);
      asm volatile("" : "+v"(rofs[ks]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      tofs[db][0] = lds + (unsigned)(chunk_offset<D>(trow, col >> 3) + 2 * (col & 7));
      tofs[db][1] = lds + (unsigned)(chunk_offset<D>(trow + 4, col >> 3) + 2 * (col & 7));
      asm volatile("" : "+v"(tofs[db][0]), "+v"(tofs[db][1]));
    }
  }
  static_assert((kStages - 1) * kStage + kTile + 16 * 2 * D < 65536, "stage offsets must fit the ds_read immediate");
  auto rd_row = [&](unsigned off, int ks) -> bf16x8_t {
    return *(const LDS_AS bf16x8_t*)(uintptr_t)(rofs[ks] + off);
  };
  auto rd_tr = [&](unsigned off, int db) -> bf16x8_t {
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(uintptr_t)(tofs[db][0] + off));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(uintptr_t)(tofs[db][1] + off));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4,
                                   5, 6, 7);
  };
  // The hand-over buffer of a pair: lane l's 16 values as four 16-byte chunks, chunk
  // j at (j * 64 + l) * 16, so each 16-byte access of a wave covers 1 KB in order.
  const unsigned xbase = (unsigned)(uintptr_t)(LDS_AS char*)xch + (unsigned)(pair * kX + lane * 16);
  auto xchg = [&](int u) -> LDS_AS f32x4_t* { return (LDS_AS f32x4_t*)(uintptr_t)(xbase + (unsigned)((u & 1) * 4 * kX)); };

  // One step s of the P role: tile u = s + 1 in stage J. Loads of tile s + 3 go to
  // the stage tile s - 1 used (last read by the dS role in step s - 1). Each phase's
  // LDS reads are issued together ahead of the products that take them (the
  // scheduling barriers keep the compiler from spreading them out again, one read
  // in front of each product).
  auto step_p = [&](auto j_tag, int s) {
    constexpr int J = decltype(j_tag)::value;
    constexpr unsigned CUR = J * kStage;
    const int u = s + 1;
    if (u < T) {
      bf16x8_t r[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) r[ks] = rd_row(CUR, ks);
      const LDS_AS float* l2v = (const LDS_AS float*)(uintptr_t)(lds + CUR + 2 * kTile);
      f32x4_t l4[4];
#pragma unroll
      for (int part = 0; part < 4; ++part) l4[part] = *(const LDS_AS f32x4_t*)(l2v + acc_row(4 * part, g));
      issue(s + 3, lds + (unsigned)(((J + 2) % kStages) * kStage));
      __builtin_amdgcn_sched_barrier(0);
      f32x16_t sv = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sv = mfma(r[ks], kv[ks], sv);
      bf16x8_t tr[DB][2];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        tr[db][0] = rd_tr(CUR + kTile, db);
        tr[db][1] = rd_tr(CUR + kTile + 16 * 2 * D, db);
      }
      __builtin_amdgcn_sched_barrier(0);
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c, -l4[i / 4][i % 4]));
      LDS_AS f32x4_t* x = xchg(u);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[64 * j] = f32x4_t{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
      const bf16x8_t p0 = pack8(p), p1 = pack8(p + 8);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        acc[db] = mfma(tr[db][0], p0, acc[db]);
        acc[db] = mfma(tr[db][1], p1, acc[db]);
      }
      // The hand-over writes must be done before the barrier that lets the partner
      // read them, and every read of the tile before the barrier after which its
      // stage is refilled (the barrier itself does not wait for LDS operations).
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
      issue(s + 3, lds + (unsigned)(((J + 2) % kStages) * kStage));
    }
    // Tile s + 2 has landed (the P role reads it from the next step on); tile s + 3
    // may stay in flight. The barrier also publishes this step's P to the partner.
    tile_barrier<kPerTile>();
  };
  // One step s of the dS role: tile s in stage J.
  auto step_ds = [&](auto j_tag, int s) {
    constexpr int J = decltype(j_tag)::value;
    constexpr unsigned CUR = J * kStage;
    bf16x8_t r[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) r[ks] = rd_row(CUR + kTile, ks);
    const LDS_AS float* dvv = (const LDS_AS float*)(uintptr_t)(lds + CUR + 2 * kTile + 256);
    const LDS_AS f32x4_t* x = xchg(s);
    f32x4_t d4[4], p4[4];
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      d4[part] = *(const LDS_AS f32x4_t*)(dvv + acc_row(4 * part, g));
      p4[part] = x[64 * part];
    }
    issue(s + 3, lds + (unsigned)(((J + 3) % kStages) * kStage));
    __builtin_amdgcn_sched_barrier(0);
    f32x16_t dp = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dp = mfma(r[ks], kv[ks], dp);
    bf16x8_t tr[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      tr[db][0] = rd_tr(CUR, db);
      tr[db][1] = rd_tr(CUR + 16 * 2 * D, db);
    }
    __builtin_amdgcn_sched_barrier(0);
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ds[i] = p4[i / 4][i % 4] * (dp[i] - d4[i / 4][i % 4]);
    const bf16x8_t s0 = pack8(ds), s1 = pack8(ds + 8);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma(tr[db][0], s0, acc[db]);
      acc[db] = mfma(tr[db][1], s1, acc[db]);
    }
    // Every read of this tile must be done before the barrier after which its stage
    // is refilled (the products that take the read values may still follow it).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    tile_barrier<kPerTile>();  // as in step_p
  };
  static_assert(kStages == 4, "the unrolled loops below cover a ring of four stages");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  issue(0, lds);
  issue(1, lds + (unsigned)kStage);
  tile_barrier<kPerTile>();  // tile 0 landed; tile 1 may stay in flight
  // Step -1: the P role takes tile 0; the dS role only loads and waits.
  if (role_p) {
    step_p(I0{}, -1);
    int s = 0;
    for (; s + kStages <= T; s += kStages) {
      step_p(I1{}, s);
      step_p(I2{}, s + 1);
      step_p(I3{}, s + 2);
      step_p(I0{}, s + 3);
    }
    if (s < T) step_p(I1{}, s);
    if (s + 1 < T) step_p(I2{}, s + 1);
    if (s + 2 < T) step_p(I3{}, s + 2);
  } else {
    issue(2, lds + (unsigned)(2 * kStage));
    tile_barrier<kPerTile>();
    int s = 0;
    for (; s + kStages <= T; s += kStages) {
      step_ds(I0{}, s);
      step_ds(I1{}, s + 1);
      step_ds(I2{}, s + 2);
      step_ds(I3{}, s + 3);
    }
    if (s < T) step_ds(I0{}, s);
    if (s + 1 < T) step_ds(I1{}, s + 1);
    if (s + 2 < T) step_ds(I2{}, s + 2);
  }
  // Loads issued past the last tile (zero fills) must land before the workgroup's
  // LDS can be handed to another workgroup.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (krow < N) {
    __bf16* out = (role_p ? dv : dk) + head + (size_t)krow * D;
    const float f = role_p ? 1.0f : scale;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = db * 32 + 8 * i4 + 4 * g;
        const f32x2_t a = {acc[db][4 * i4] * f, acc[db][4 * i4 + 1] * f};
        const f32x2_t b = {acc[db][4 * i4 + 2] * f, acc[db][4 * i4 + 3] * f};
        *(u32x2_t*)(out + col) = u32x2_t{__builtin_bit_cast(unsigned, __builtin_convertvector(a, bf16x2_t)),
                                         __builtin_bit_cast(unsigned, __builtin_convertvector(b, bf16x2_t))};
      }
    }
  }
}

template <int D>
void launch_bwd_d(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                  void* dq, void* dk, void* dv, int BH, int N, float scale, float* dvec, float* lse2, hipStream_t st) {
  const long long rows = (long long)BH * N;
  constexpr int kRowsPerBlock = 4 * (64 / (D / 8));
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256), 0,
                     st, (const __bf16*)o, (const __bf16*)dO, lse, dvec, lse2, rows);
  const int tiles = (N + 127) / 128;
  const int total = BH * tiles;
  const float c = scale * kLog2e;
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)total), dim3(256), 0, st, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, (const __bf16*)dO, dvec, lse2, (__bf16*)dq, N, tiles, total, c, scale);
  if constexpr (D == 128) {
    hipLaunchKernelGGL(bwd_dkdv_pair_kernel<D>, dim3((unsigned)total), dim3(512), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, dvec, lse2, (__bf16*)dk, (__bf16*)dv, N,
                       tiles, total, c, scale);
  } else {
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)total), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, dvec, lse2, (__bf16*)dk, (__bf16*)dv, N,
                       tiles, total, c, scale);
  }
}

}  // namespace

int launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
               void* dk, void* dv, int B, int H, int N, int d, float scale, void* workspace, void* stream) {
  const int BH = B * H;
  float* dvec = (float*)workspace;
  float* lse2 = dvec + (size_t)BH * N;
  hipStream_t st = (hipStream_t)stream;
  if (d == 128) launch_bwd_d<128>(q, k, v, o, lse, dO, dq, dk, dv, BH, N, scale, dvec, lse2, st);
  else launch_bwd_d<64>(q, k, v, o, lse, dO, dq, dk, dv, BH, N, scale, dvec, lse2, st);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
