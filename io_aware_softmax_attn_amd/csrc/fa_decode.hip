// Decode-shaped attention forward on gfx950: a few query rows per head (Nq <= 16)
// against a long key/value sequence (Nk keys), the workload the KP page contrasts
// with prefill (sections 常见误区 and 自测题: decode is bound by memory traffic,
// not by arithmetic). Per key the work is 4*Nq*d flops against 4*d bytes of K and
// V, at most 16 flops per byte, far below the matrix cores' ridge, so this path is
// written for HBM bandwidth: coalesced 16-byte row loads and enough independent
// workgroups in flight. One query row runs its dot products and PV sum on the
// vector ALUs in fp32; 2 to 16 rows run them on the matrix cores (the vector issue
// slots run out first there).
//
// The key range of each (b, h) is split into chunks, one workgroup per chunk
// (kernel 1), whose partial results are merged afterwards (kernel 2):
//   kernel 1  per chunk s: O_s = softmax over the chunk's keys applied to V
//             (fp32, normalised) and LSE_s (log2 units), into the workspace;
//   kernel 2  per query row: the FA1 page's update (derivation steps 2 and 4-5)
//             over whole chunks, m = max_s LSE_s,
//             L = m + log2 sum_s 2^(LSE_s - m),  O = sum_s 2^(LSE_s - L) O_s,
//             then O to bf16 (nearest-even) and LSE = ln2 * L.
// Inside a chunk each wave runs the online softmax (same page, steps 1-5) over
// batches of keys; the waves' states are merged through LDS at the end.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {

// The partial results of fa_decode_fwd_noalloc: a fixed array in device memory, one
// per GPU, held until the process ends. In host code `scratch` names a host-side
// stand-in, not the device array: host code only ever uses the address that
// decode_scratch() looks up for the current device.
static __device__ __attribute__((used)) __align__(256) unsigned char scratch[FA_DECODE_SCRATCH_BYTES];

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Lane layout of one wave's row loads: a K or V row of D bf16 is kLanesPerKey
// 16-byte pieces, so one 64-lane load covers kGroups consecutive rows (1 KB at
// D = 128, fully coalesced); lane l holds piece l % kLanesPerKey of row l / kLanesPerKey.
template <int D>
struct DecCfg {
  static constexpr int kLanesPerKey = D / 8;
  static constexpr int kGroups = 64 / kLanesPerKey;
  static constexpr int kLoads = 4;                      // row loads per wave per batch
  static constexpr int kWaveKeys = kLoads * kGroups;    // keys per wave per batch
  static constexpr int kBlockKeys = 4 * kWaveKeys;      // keys per workgroup per batch
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over the kLanesPerKey lanes of one row (all lanes get the same value: each
// step adds two partial sums that are equal as a set, and fp32 addition is
// commutative).
template <int D>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: pairs
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: quads
  x += dpp<0x141>(x);  // row_half_mirror: the two quads of each 8 lanes
  if constexpr (D == 128) x += dpp<0x140>(x);  // row_mirror: the two halves of each 16 lanes
  return x;
}

__device__ __forceinline__ f32x2_t swap16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return f32x2_t{__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}
__device__ __forceinline__ f32x2_t swap32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return f32x2_t{__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}

// Combine the kGroups row groups of a wave: lanes holding the same piece index in
// different groups. Every lane ends with the same result.
template <int D>
__device__ __forceinline__ float groups_sum(float x) {
  if constexpr (D == 64) x += dpp<0x128>(x);  // row_ror:8, the two 8-lane groups of a row
  f32x2_t r = swap16(x);
  x = r[0] + r[1];
  r = swap32(x);
  return r[0] + r[1];
}
template <int D>
__device__ __forceinline__ float groups_max(float x) {
  if constexpr (D == 64) x = fmaxf(x, dpp<0x128>(x));
  f32x2_t r = swap16(x);
  x = fmaxf(r[0], r[1]);
  r = swap32(x);
  return fmaxf(r[0], r[1]);
}

// Dot product of 8 bf16 pairs, fp32 accumulation. Each vector element is copied
// to a scalar before the bit cast: a bit cast applied to an element of an
// ext_vector_type value directly reads element 0 for every index with this
// compiler.
__device__ __forceinline__ float dot8(const u32x4_t& a, const u32x4_t& b) {
  float d = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned aj = a[j], bj = b[j];
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, aj), __builtin_bit_cast(bf16x2_t, bj), d, false);
  }
  return d;
}

// Kernel 1. Workgroup (bh, s) covers keys [s*chunk, min((s+1)*chunk, Nk)) of head
// bh for all Nq query rows (NQ >= Nq is the compiled row count; rows >= Nq are
// zero and never stored). Wave w takes keys base + w*kWaveKeys + u*kGroups + g of
// each batch; keys past the chunk's end are masked (score -inf), and their loads
// read row min(key, Nk-1), which is inside the head. Writes part_o[bh][s][i][:]
// (fp32, normalised over the chunk) and part_lse[bh][s][i] (log2 units).
template <int D, int NQ>
__global__ void __launch_bounds__(256) dec_split_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                        const __bf16* __restrict__ v, float* __restrict__ part_o,
                                                        float* __restrict__ part_lse, int Nq, int Nk, int chunk,
                                                        int S, float c) {
  using C = DecCfg<D>;
  constexpr int L = C::kLoads;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = lane % C::kLanesPerKey, g = lane / C::kLanesPerKey;
  const int s = blockIdx.x % S;
  const size_t bh = blockIdx.x / S;
  const int k0 = s * chunk;
  const int k1 = min(k0 + chunk, Nk);

  u32x4_t qv[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    qv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (i < Nq) qv[i] = *(const u32x4_t*)(q + (bh * Nq + i) * D + 8 * t);
  }
  float m[NQ], l[NQ], acc[NQ][8];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    m[i] = -__builtin_inff();
    l[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  }

  const __bf16* kh = k + bh * (size_t)Nk * D + 8 * t;
  const __bf16* vh = v + bh * (size_t)Nk * D + 8 * t;
  const int wkey0 = wave * C::kWaveKeys + g;  // this lane's key offset inside a batch, load 0
  auto load = [&](int base, u32x4_t (&kr)[L], u32x4_t (&vr)[L]) {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const size_t row = (size_t)min(base + wkey0 + u * C::kGroups, Nk - 1);
      kr[u] = __builtin_nontemporal_load((const u32x4_t*)(kh + row * D));
      vr[u] = __builtin_nontemporal_load((const u32x4_t*)(vh + row * D));
    }
  };
  auto process = [&](int base, const u32x4_t (&kr)[L], const u32x4_t (&vr)[L]) {
    float sc[L][NQ];
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const bool live = base + wkey0 + u * C::kGroups < k1;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const float d = row_sum<D>(dot8(kr[u], qv[i]));
        sc[u][i] = live ? d * c : -__builtin_inff();
      }
    }
    float p[L][NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      float bm = sc[0][i];
#pragma unroll
      for (int u = 1; u < L; ++u) bm = fmaxf(bm, sc[u][i]);
      bm = groups_max<D>(bm);
      const float mn = fmaxf(m[i], bm);
      const float ms = mn == -__builtin_inff() ? 0.0f : mn;  // no key yet: keep every term at 0
      const float alpha = __builtin_amdgcn_exp2f(m[i] - ms);
      m[i] = mn;
      float ls = l[i] * alpha;
#pragma unroll
      for (int u = 0; u < L; ++u) {
        p[u][i] = __builtin_amdgcn_exp2f(sc[u][i] - ms);
        ls += p[u][i];
      }
      l[i] = ls;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < L; ++u) {
      float vf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // bf16 pair -> two fp32 (bf16 is the top half of fp32)
        const unsigned w = vr[u][j];
        vf[2 * j] = __builtin_bit_cast(float, w << 16);
        vf[2 * j + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
      }
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(p[u][i], vf[j], acc[i][j]);
      }
    }
  };

  // Batches of kBlockKeys keys; the next batch's rows are loaded before the
  // current one is processed.
  u32x4_t kc[L], vc[L], kn[L], vn[L];
  load(k0, kc, vc);
  for (int base = k0; base < k1; base += C::kBlockKeys) {
    const bool more = base + C::kBlockKeys < k1;
    if (more) load(base + C::kBlockKeys, kn, vn);
    process(base, kc, vc);
    if (more) {
#pragma unroll
      for (int u = 0; u < L; ++u) {
        kc[u] = kn[u];
        vc[u] = vn[u];
      }
    }
  }

  // Each group of lanes summed its own keys; the wave's state is the sum over groups
  // (m is already wave-wide).
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    l[i] = groups_sum<D>(l[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = groups_sum<D>(acc[i][j]);
  }

  // Merge the four waves' states (m_w, l_w, acc_w) through LDS.
  __shared__ float sm[4][NQ], sl[4][NQ];
  __shared__ float so[4][NQ][D];
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      sm[wave][i] = m[i];
      sl[wave][i] = l[i];
    }
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) so[wave][i][8 * t + j] = acc[i][j];
    }
  }
  __syncthreads();
  const size_t out_row0 = (bh * S + s) * (size_t)Nq;
  for (int e = threadIdx.x; e < Nq * D; e += 256) {
    const int i = e / D, col = e % D;
    float mx = sm[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, sm[w][i]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = __builtin_amdgcn_exp2f(sm[w][i] - mx);  // 0 for a wave that saw no key
      den = __builtin_fmaf(a, sl[w][i], den);
      num = __builtin_fmaf(a, so[w][i][col], num);
    }
    part_o[(out_row0 + i) * D + col] = num / den;
    if (col == 0) part_lse[out_row0 + i] = mx + __builtin_log2f(den);
  }
}

// Kernel 1 for 2 to 16 query rows, on the matrix cores. With more query rows the
// VALU kernel above runs out of vector issue slots before HBM runs out of bytes
// (four dot2, four DPP adds, an exp2 and eight FMAs per key and query: 4.4 TB/s at
// 8 rows, 2.0 at 16); this kernel streams at the same rate for every row count,
// and from 2 rows on at least as fast as the VALU kernel. The query rows are padded
// to 16 and both products run as v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T   (16 keys x 16 queries per product, 32 of d per k-step);
//   O^T += V^T P^T (16 of d x 16 queries per product, 32 keys per k-step).
// Each wave streams its own 32-key tiles of the chunk (tiles w, w+4, ...). K rows
// are loaded straight into the A operands (lane l: key l%16, d 8*(l/16)..+8 of a
// k-step); V rows are loaded coalesced, written to the wave's own LDS tile and read
// back transposed with ds_read_b64_tr_b16. A lane holds scores of keys 4G+i and
// 16+4G+i (G = l/16) for query l%16; the V^T operand reads use the same key order,
// so the contraction pairs each P with its V row. The online softmax is the FA1
// page's update per 32-key tile (steps 1-5) with the exact running max. P enters
// the PV product as two bf16 terms, P = hi + lo with lo = bf16(P - hi), so the sum
// keeps about 16 significant bits of P, like the fp32 P of the VALU kernel; the
// matrix cores have the slots to spare, as this path is bound by HBM.
template <int D>
struct MfmaDecCfg {
  static constexpr int kTileKeys = 32;                      // keys per wave per step
  static constexpr int kKS = D / 32;                        // k-steps of S^T = K Q^T
  static constexpr int kDB = D / 16;                        // 16-row d-blocks of O^T
  static constexpr int kChunks = D / 8;                     // 16-byte chunks per K/V row
  static constexpr int kRowsPerLoad = 64 / kChunks;         // rows one wave-wide 16-byte load covers
  static constexpr int kVLoads = kTileKeys / kRowsPerLoad;  // V row loads per lane per tile
  static constexpr int kTileBytes = kTileKeys * 2 * D;      // one wave's V tile in LDS
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
#define FA_LDS_AS __attribute__((address_space(3)))

// XOR swizzle of the 16-byte chunk index of V tile row r (a key). A transposing read
// by 16 lanes covers 4 consecutive rows x 2 adjacent chunks (an even chunk and the
// next); the even XOR values 2*(r%4) send the 4 rows to 8 distinct chunks, so the
// 16 lanes hit 8 distinct 16-byte bank groups. At D = 128 bit 2 of the row also
// selects the other half of the row, separating neighbouring lane groups.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  int x = 2 * (r & 3);
  if constexpr (D == 128) x |= 8 * ((r >> 2) & 1);
  return x;
}

// Max and sum over the four lanes l%16 + 16*G (G = 0..3) that hold one query.
__device__ __forceinline__ float qmax4(float x) {
  f32x2_t r = swap16(x);
  x = fmaxf(r[0], r[1]);
  r = swap32(x);
  return fmaxf(r[0], r[1]);
}
__device__ __forceinline__ float qsum4(float x) {
  f32x2_t r = swap16(x);
  x = r[0] + r[1];
  r = swap32(x);
  return r[0] + r[1];
}

template <int D>
__global__ void __launch_bounds__(256, 2) dec_split_mfma_kernel(const __bf16* __restrict__ q,
                                                                const __bf16* __restrict__ k,
                                                                const __bf16* __restrict__ v,
                                                                float* __restrict__ part_o,
                                                                float* __restrict__ part_lse, int Nq, int Nk,
                                                                int chunk, int S, float c) {
  using C = MfmaDecCfg<D>;
  constexpr int KS = C::kKS, DB = C::kDB, VL = C::kVLoads;
  // The waves' V tiles during the loop; the waves' partial O^T ([4][16][D] fp32, the
  // same 256*D bytes) for the merge after it.
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * C::kTileBytes];
  __shared__ float sm[4][16], sl[4][16];
  static_assert(4 * C::kTileBytes == 4 * 16 * D * 4, "partial O^T must fit the V tiles");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = lane >> 4, j = lane & 15;
  const int s = blockIdx.x % S;
  const size_t bh = blockIdx.x / S;
  const int k0 = s * chunk;
  const int k1 = min(k0 + chunk, Nk);
  const int ntiles = (k1 - k0 + C::kTileKeys - 1) / C::kTileKeys;

  // Q^T operands: lane l holds query l%16 (zero past Nq), d 32*ks + 8*(l/16) .. +8.
  bf16x8_t qB[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qB[ks] = bf16x8_t{};
    if (j < Nq) qB[ks] = *(const bf16x8_t*)(q + (bh * Nq + j) * D + 32 * ks + 8 * G);
  }
  const __bf16* kh = k + bh * (size_t)Nk * D;
  const __bf16* vh = v + bh * (size_t)Nk * D;
  const unsigned stage = (unsigned)(uintptr_t)(FA_LDS_AS unsigned char*)smem + (unsigned)(wave * C::kTileBytes);
  // This lane's LDS byte offsets: its V row writes, and its transposing reads of
  // d-block db, k-slot half r (keys 16r + 4G + 0..3, column 16db + j).
  unsigned vw[VL], vr[DB][2];
#pragma unroll
  for (int u = 0; u < VL; ++u) {
    const int row = u * C::kRowsPerLoad + lane / C::kChunks, ch = lane % C::kChunks;
    vw[u] = stage + (unsigned)(row * 2 * D + ((ch ^ vswz<D>(row)) << 4));
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 16 * r + 4 * G + (j >> 2), dcol = 16 * db + 4 * (j & 3);
      vr[db][r] = stage + (unsigned)(row * 2 * D + (((dcol >> 3) ^ vswz<D>(row)) << 4) + 2 * (dcol & 7));
    }
  }

  float m = -__builtin_inff(), lsum = 0.0f;
  f32x4_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4_t{};

  // Tile t of the chunk: keys k0 + 32t ..; rows past Nk read row Nk-1 (inside the
  // head) and are masked.
  auto load = [&](int t, u32x4_t (&kr)[2][KS], u32x4_t (&vrow)[VL]) {
    const int key0 = k0 + t * C::kTileKeys;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const size_t key = (size_t)min(key0 + 16 * b + j, Nk - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kr[b][ks] = __builtin_nontemporal_load((const u32x4_t*)(kh + key * D + 32 * ks + 8 * G));
    }
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      const size_t row = (size_t)min(key0 + u * C::kRowsPerLoad + lane / C::kChunks, Nk - 1);
      vrow[u] = __builtin_nontemporal_load((const u32x4_t*)(vh + row * D + 8 * (lane % C::kChunks)));
    }
  };
  auto process = [&](int t, const u32x4_t (&kr)[2][KS], const u32x4_t (&vrow)[VL]) {
    // V rows into this wave's tile (the wave's own LDS accesses run in order, so the
    // transposing reads below see them, and the previous tile's reads are done).
#pragma unroll
    for (int u = 0; u < VL; ++u) *(FA_LDS_AS u32x4_t*)(uintptr_t)vw[u] = vrow[u];
    f32x4_t sc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sc[b] = f32x4_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[b][ks]), qB[ks], sc[b], 0, 0,
                                                        0);
    }
    const int key0 = k0 + t * C::kTileKeys;
    float tv[2][4];
    float mt = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = key0 + 16 * b + 4 * G + i < k1;
        tv[b][i] = live ? sc[b][i] * c : -__builtin_inff();
        mt = fmaxf(mt, tv[b][i]);
      }
    }
    // Steps 1-2: the tile's row max (every tile holds a live key, so it is finite),
    // the new running max and the factor for the old state.
    const float mn = fmaxf(m, qmax4(mt));
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    bf16x8_t phi, plo;
    float ps = 0.0f;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(tv[b][i] - mn);
        ps += p;
        const __bf16 hi = (__bf16)p;
        phi[4 * b + i] = hi;
        plo[4 * b + i] = (__bf16)(p - (float)hi);
      }
    }
    lsum = __builtin_fmaf(lsum, alpha, ps);
    // Steps 3-5: rescale the accumulator and add P V for this tile.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] *= alpha;
      const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS_AS i16x4_t*)(uintptr_t)vr[db][0]);
      const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS_AS i16x4_t*)(uintptr_t)vr[db][1]);
      const bf16x8_t va = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo4), __builtin_bit_cast(bf16x4_t, hi4),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[db], 0, 0, 0);
    }
  };

  // This wave's tiles (wave, wave + 4, ...) alternate between two register buffers:
  // the next tile's rows are loaded into one while the other is processed, and no
  // tile is copied from one buffer to the other (a copy would wait for the loads
  // just issued). The first tile is waited for here, before the loop.
  u32x4_t ka[2][KS], va[VL], kb[2][KS], vb[VL];
  if (wave < ntiles) {
    load(wave, ka, va);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(ka[b][ks]));
    }
#pragma unroll
    for (int u = 0; u < VL; ++u) asm volatile("" : "+v"(va[u]));
  }
  int t = wave;
  for (; t + 4 < ntiles; t += 8) {
    load(t + 4, kb, vb);
    process(t, ka, va);
    if (t + 8 < ntiles) load(t + 8, ka, va);
    process(t + 4, kb, vb);
  }
  if (t < ntiles) process(t, ka, va);

  // A lane's sum covers its own keys; the query's sum adds the four lanes holding it.
  lsum = qsum4(lsum);
  __syncthreads();  // every wave is done with its V tile: the LDS now holds partial O^T
  float* so = (float*)smem;
  if (G == 0) {
    sm[wave][j] = m;
    sl[wave][j] = lsum;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) so[(wave * 16 + j) * D + 16 * db + 4 * G + i] = acc[db][i];
  }
  __syncthreads();
  const size_t out_row0 = (bh * S + s) * (size_t)Nq;
  for (int e = threadIdx.x; e < Nq * D; e += 256) {
    const int i = e / D, col = e % D;
    float mx = sm[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, sm[w][i]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = __builtin_amdgcn_exp2f(sm[w][i] - mx);  // 0 for a wave that saw no key
      den = __builtin_fmaf(a, sl[w][i], den);
      num = __builtin_fmaf(a, so[(w * 16 + i) * D + col], num);
    }
    part_o[(out_row0 + i) * D + col] = num / den;
    if (col == 0) part_lse[out_row0 + i] = mx + __builtin_log2f(den);
  }
}

// Kernel 2: one wave per query row (b, h, i); lane l owns columns D/64*l .. +D/64-1.
template <int D>
__global__ void __launch_bounds__(256) dec_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_lse, __bf16* __restrict__ o,
                                                        float* __restrict__ lse, int rows, int Nq, int S) {
  constexpr int kCols = D / 64;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (size_t)rows) return;
  const int lane = threadIdx.x & 63;
  const size_t bh = row / Nq;
  const int i = (int)(row % Nq);
  const float* pl = part_lse + bh * S * (size_t)Nq + i;
  float mx = -__builtin_inff();
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, pl[(size_t)s * Nq]);
  float den = 0.0f, acc[kCols] = {};
  for (int s = 0; s < S; ++s) {
    const float w = __builtin_amdgcn_exp2f(pl[(size_t)s * Nq] - mx);
    den += w;
    const float* po = part_o + ((bh * S + s) * Nq + i) * D + kCols * lane;
#pragma unroll
    for (int j = 0; j < kCols; ++j) acc[j] = __builtin_fmaf(w, po[j], acc[j]);
  }
  const float inv = 1.0f / den;
  __bf16* orow = o + row * D + kCols * lane;
  if constexpr (kCols == 2) {
    *(bf16x2_t*)orow = __builtin_convertvector((f32x2_t){acc[0] * inv, acc[1] * inv}, bf16x2_t);
  } else {
    orow[0] = (__bf16)(acc[0] * inv);
  }
  if (lane == 0) lse[row] = kLn2 * (mx + __builtin_log2f(den));
}

template <int D, int NQ>
void launch_split(const void* q, const void* k, const void* v, float* po, float* pl, int BH, int Nq, int Nk,
                  const DecodePlan& p, float c, hipStream_t st) {
  hipLaunchKernelGGL((dec_split_kernel<D, NQ>), dim3((unsigned)(BH * p.splits)), dim3(256), 0, st,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, po, pl, Nq, Nk, p.chunk, p.splits, c);
}

template <int D>
void launch_split_d(const void* q, const void* k, const void* v, float* po, float* pl, int BH, int Nq, int Nk,
                    const DecodePlan& p, float c, hipStream_t st) {
  if (Nq <= 1) launch_split<D, 1>(q, k, v, po, pl, BH, Nq, Nk, p, c, st);
  else
    hipLaunchKernelGGL((dec_split_mfma_kernel<D>), dim3((unsigned)(BH * p.splits)), dim3(256), 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, po, pl, Nq, Nk, p.chunk, p.splits, c);
}

}  // namespace

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

int decode_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Once per device, with that device current: its copy of the array has its own address.
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return FA_OK;
}

int launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int d, float scale, void* workspace, void* stream) {
  const DecodePlan p = decode_plan(B, H, Nq, Nk, d);
  const int BH = B * H;
  float* po = (float*)workspace;
  float* pl = po + (size_t)BH * p.splits * Nq * d;
  const float c = scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  const int rows = BH * Nq;
  const unsigned merge_blocks = (unsigned)((rows + 3) / 4);
  if (d == 128) {
    launch_split_d<128>(q, k, v, po, pl, BH, Nq, Nk, p, c, st);
    hipLaunchKernelGGL(dec_merge_kernel<128>, dim3(merge_blocks), dim3(256), 0, st, po, pl, (__bf16*)o, lse, rows,
                       Nq, p.splits);
  } else {
    launch_split_d<64>(q, k, v, po, pl, BH, Nq, Nk, p, c, st);
    hipLaunchKernelGGL(dec_merge_kernel<64>, dim3(merge_blocks), dim3(256), 0, st, po, pl, (__bf16*)o, lse, rows, Nq,
                       p.splits);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
