// Internal interface between the host API (fa_api.cpp, plain C++) and the HIP
// translation units that own the kernels. No HIP types appear here so that the
// API layer builds with any host compiler.
#pragma once
#include <cstddef>
#include <cstdint>

namespace fa {

// Tile shape chosen for a problem; filled in by select_blocks.
struct Blocks {
  int br;      // query rows per workgroup
  int bc;      // keys per K/V tile
  int nwaves;  // 64-lane waves per workgroup
};

// Picks the fused kernel's tile shape (see fa_select.cpp).
Blocks select_blocks(int d, int N, int B, int H);

// Enqueue the fused forward; returns a fa_status code. Arguments already validated.
// order: workgroup-to-tile order (0 = XCD-aware, the default; see fa_fwd_tile_order).
int launch_fused(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, const Blocks& blk, void* stream, int order = 0);

// Enqueue the three unfused kernels; returns a fa_status code.
int launch_unfused(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, void* workspace, void* stream);

// Key-range split of the decode-shaped forward (see fa_select.cpp).
struct DecodePlan {
  int splits;  // chunks per (b, h), one workgroup each
  int chunk;   // keys per chunk (the last chunk of a head may be shorter)
};
DecodePlan decode_plan(int B, int H, int Nq, int Nk, int d);

// Enqueue the decode split and merge kernels; returns a fa_status code. Arguments
// already validated; workspace holds at least fa_decode_workspace_bytes.
int launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int d, float scale, void* workspace, void* stream);

// Device address, on the current device, of the decode path's fixed scratch array
// (FA_DECODE_SCRATCH_BYTES), looked up once per device; returns a fa_status code.
int decode_scratch(void** ptr);

// Enqueue the three backward kernels; returns a fa_status code. Arguments already
// validated; workspace holds at least fa_bwd_workspace_bytes(B, H, N).
int launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
               void* dk, void* dv, int B, int H, int N, int d, float scale, void* workspace, void* stream);

// 1 if the current device is gfx950, 0 if not, negative fa_status on HIP error.
int device_is_gfx950();

}  // namespace fa
