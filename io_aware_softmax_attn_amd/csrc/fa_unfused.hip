// The textbook three-kernel attention forward on gfx950, kept only as a traffic
// and error baseline for the fused kernel ("01 · 注意力为什么是 IO 瓶颈", section 3
// table and section 5 ``naive_attention``): each step stores its N x N result in
// device memory and the next step reads it back.
//   kernel 1  S = scale * Q K^T            fp32 [B,H,N,Ns]   (Ns = N rounded up to 64)
//   kernel 2  P = softmax(S) row by row    bf16 [B,H,N,Ns]   and LSE fp32 [B,H,N]
//   kernel 3  O = P V                      bf16 [B,H,N,d]
// P is stored as a 16-bit type, as the pages' fused kernel converts it before the
// PV product (same page, section 6). Both products use v_mfma_f32_32x32x16_bf16.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

__host__ __device__ constexpr int padded(int n) { return (n + 63) / 64 * 64; }

// Kernel 1: one workgroup computes a 128 x 64 block of S; wave w owns rows
// 32w..32w+31 of it and both 32-key blocks. Operands come straight from global
// memory (16-byte loads); rows/keys past N read as zero and are not stored.
template <int D>
__global__ void __launch_bounds__(256) unf_qk_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                     float* __restrict__ s, int N, float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  const int bh = blockIdx.z;
  const int Ns = padded(N);
  const int i0 = blockIdx.y * 128 + wave * 32;
  const int j0 = blockIdx.x * 64;
  const size_t head = (size_t)bh * N * D;
  const int qrow = i0 + (lane & 31);
  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    bf16x8_t a = bf16x8_t{};
    if (qrow < N) a = *(const bf16x8_t*)(q + head + (size_t)qrow * D + ks * 16 + g * 8);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int krow = j0 + nb * 32 + (lane & 31);
      bf16x8_t b = bf16x8_t{};
      if (krow < N) b = *(const bf16x8_t*)(k + head + (size_t)krow * D + ks * 16 + g * 8);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[nb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int col = j0 + nb * 32 + (lane & 31);
    if (col >= N) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = i0 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (row < N) s[((size_t)bh * N + row) * Ns + col] = acc[nb][i] * scale;
    }
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Kernel 2: one wave per row. Pass 1 reads the row and forms the max and the sum
// of exp(s - max); pass 2 reads it again and writes P = exp(s - max) / sum as bf16
// (zeros in the padding columns N..Ns-1) and LSE = max + ln(sum).
__global__ void __launch_bounds__(256) unf_softmax_kernel(const float* __restrict__ s, __bf16* __restrict__ p,
                                                          float* __restrict__ lse, long long rows, int N) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int Ns = padded(N);
  const float* srow = s + (size_t)row * Ns;
  float m = -__builtin_inff();
  for (int j = lane; j < N; j += 64) m = fmaxf(m, srow[j]);
  m = wave_max(m);
  float l = 0.0f;
  for (int j = lane; j < N; j += 64) l += expf(srow[j] - m);
  l = wave_sum(l);
  const float inv = 1.0f / l;
  __bf16* prow = p + (size_t)row * Ns;
  for (int j = lane; j < Ns; j += 64) prow[j] = (__bf16)(j < N ? expf(srow[j] - m) * inv : 0.0f);
  if (lane == 0) lse[row] = m + logf(l);
}

// Kernel 3: one workgroup computes 128 query rows x all of d; wave w owns 32 rows.
// V is staged through LDS 64 keys at a time and read as the B operand with
// ds_read_b64_tr_b16; P is read from global memory as the A operand (16 bytes of
// one row per lane). Keys past N have P = 0 and V = 0.
template <int D>
__global__ void __launch_bounds__(256) unf_pv_kernel(const __bf16* __restrict__ p, const __bf16* __restrict__ v,
                                                     __bf16* __restrict__ o, int N) {
  __shared__ __attribute__((aligned(16))) __bf16 vs[64 * D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  const int bh = blockIdx.y;
  const int Ns = padded(N);
  const int i0 = blockIdx.x * 128 + wave * 32;
  const int qrow = i0 + (lane & 31);
  const __bf16* prow = p + ((size_t)bh * N + (size_t)min(qrow, N - 1)) * Ns;
  const __bf16* vh = v + (size_t)bh * N * D;
  f32x16_t acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16_t{};
  for (int k0 = 0; k0 < N; k0 += 64) {
    __syncthreads();
    for (int c = threadIdx.x; c < 64 * D / 8; c += 256) {
      const int r = c / (D / 8), cc = c % (D / 8);
      bf16x8_t x = bf16x8_t{};
      if (k0 + r < N) x = *(const bf16x8_t*)(vh + (size_t)(k0 + r) * D + cc * 8);
      *(bf16x8_t*)(vs + r * D + cc * 8) = x;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t a = *(const bf16x8_t*)(prow + k0 + ks * 16 + g * 8);
      if (qrow >= N) a = bf16x8_t{};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int dcol = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int r0 = ks * 16 + 8 * g + ((lane & 15) >> 2);
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(LDS_AS __bf16*)(vs + r0 * D + dcol));
        const i16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(LDS_AS __bf16*)(vs + (r0 + 4) * D + dcol));
        const bf16x8_t b = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi), 0,
                                                   1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[db], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = i0 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (row < N) o[((size_t)bh * N + row) * D + db * 32 + (lane & 31)] = (__bf16)acc[db][i];
    }
  }
}

template <int D>
int launch_unfused_d(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                     float scale, void* workspace, hipStream_t st) {
  const int Ns = padded(N);
  const long long BH = (long long)B * H;
  float* s = (float*)workspace;
  __bf16* p = (__bf16*)((char*)workspace + (size_t)BH * N * Ns * 4);
  hipLaunchKernelGGL(unf_qk_kernel<D>, dim3(Ns / 64, (N + 127) / 128, (unsigned)BH), dim3(256), 0, st,
                     (const __bf16*)q, (const __bf16*)k, s, N, scale);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  const long long rows = BH * N;
  hipLaunchKernelGGL(unf_softmax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, s, p, lse, rows, N);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  hipLaunchKernelGGL(unf_pv_kernel<D>, dim3((N + 127) / 128, (unsigned)BH), dim3(256), 0, st, p,
                     (const __bf16*)v, (__bf16*)o, N);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

int launch_unfused(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, void* workspace, void* stream) {
  if ((long long)B * H > 65535) return FA_ERR_OVERFLOW;  // grid z / y limit of the unfused kernels
  hipStream_t st = (hipStream_t)stream;
  return d == 128 ? launch_unfused_d<128>(q, k, v, o, lse, B, H, N, scale, workspace, st)
                  : launch_unfused_d<64>(q, k, v, o, lse, B, H, N, scale, workspace, st);
}

}  // namespace fa
