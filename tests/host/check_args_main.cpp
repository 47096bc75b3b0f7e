// Host-only test of the C ABI's validation and dispatch layer (fa_api.cpp,
// fa_select.cpp), built with g++ under AddressSanitizer and UBSan. The HIP side
// is replaced by the stubs below: they count launches, so every rejected call can
// be shown to return before anything would be enqueued.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "../../include/fa.h"
#include "../../io_aware_softmax_attn_amd/csrc/fa_internal.h"

namespace {
int g_launches = 0;
int g_last_br = 0;  // query-tile height of the last fused launch
int g_device = 1;  // what device_is_gfx950 reports
int g_failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::printf("FAIL line %d: %s\n", line, what);
    ++g_failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)
}  // namespace

namespace fa {
int launch_fused(const void*, const void*, const void*, void*, float*, int, int, int, int, float, const Blocks& blk,
                 void*, int) {
  ++g_launches;
  g_last_br = blk.br;
  return FA_OK;
}
int launch_unfused(const void*, const void*, const void*, void*, float*, int, int, int, int, float, void*, void*) {
  ++g_launches;
  return FA_OK;
}
int launch_decode(const void*, const void*, const void*, void*, float*, int, int, int, int, int, float, void*,
                  void*) {
  ++g_launches;
  return FA_OK;
}
int launch_bwd(const void*, const void*, const void*, const void*, const float*, const void*, void*, void*, void*, int,
               int, int, int, float, void*, void*) {
  ++g_launches;
  return FA_OK;
}
int device_is_gfx950() { return g_device; }
int g_scratch_lookups = 0;
int decode_scratch(void** ptr) {
  ++g_scratch_lookups;
  static unsigned char stand_in[256];
  *ptr = stand_in;
  return FA_OK;
}
}  // namespace fa

int main() {
  // Real, aligned host buffers for a B=2 H=3 N=100 d=64 problem (never dereferenced
  // by the library; ASan would report it if they were read out of bounds).
  const int B = 2, H = 3, N = 100, d = 64;
  const size_t tb = (size_t)B * H * N * d * 2, lb = (size_t)B * H * N * 4;
  char* q = static_cast<char*>(std::aligned_alloc(256, tb));
  char* k = static_cast<char*>(std::aligned_alloc(256, tb));
  char* v = static_cast<char*>(std::aligned_alloc(256, tb));
  char* o = static_cast<char*>(std::aligned_alloc(256, tb));
  float* lse = static_cast<float*>(std::aligned_alloc(256, (lb + 255) / 256 * 256));
  const float sc = 0.125f;

  // Valid call: one launch; with a non-gfx950 device: an error and none.
  EXPECT(fa_check_args(q, k, v, o, lse, B, H, N, d, sc, 0, nullptr, 0) == FA_OK);
  EXPECT(fa_fwd(q, k, v, o, lse, B, H, N, d, sc, nullptr) == FA_OK && g_launches == 1);
  g_device = 0;
  EXPECT(fa_fwd(q, k, v, o, lse, B, H, N, d, sc, nullptr) == FA_ERR_DEVICE && g_launches == 1);
  g_device = FA_ERR_HIP;
  EXPECT(fa_fwd(q, k, v, o, lse, B, H, N, d, sc, nullptr) == FA_ERR_HIP && g_launches == 1);
  g_device = 1;

  // Every argument error returns its code and launches nothing.
  const int before = g_launches;
  EXPECT(fa_fwd(nullptr, k, v, o, lse, B, H, N, d, sc, nullptr) == FA_ERR_NULL);
  EXPECT(fa_fwd(q, k, v, o, nullptr, B, H, N, d, sc, nullptr) == FA_ERR_NULL);
  EXPECT(fa_fwd(q, k, v, o, lse, -1, H, N, d, sc, nullptr) == FA_ERR_SHAPE);
  EXPECT(fa_fwd(q, k, v, o, lse, B, H, -5, d, sc, nullptr) == FA_ERR_SHAPE);
  EXPECT(fa_fwd(q, k, v, o, lse, B, H, N, 96, sc, nullptr) == FA_ERR_HEADDIM);
  EXPECT(fa_fwd(q, k, v, o, lse, B, H, N, 0, sc, nullptr) == FA_ERR_HEADDIM);
  EXPECT(fa_fwd(q, k, v, o, lse, B, H, N, d, std::nanf(""), nullptr) == FA_ERR_SCALE);
  EXPECT(fa_fwd(q, k, v, o, lse, B, H, N, d, INFINITY, nullptr) == FA_ERR_SCALE);
  EXPECT(fa_check_args(q, k, v, o, lse, B, H, N, d, -0.5f, 0, nullptr, 0) == FA_OK);
  EXPECT(fa_fwd(q + 8, k, v, o, lse, B, H, N, d, sc, nullptr) == FA_ERR_ALIGN);
  EXPECT(fa_fwd(q, k, v, o + 2, lse, B, H, N, d, sc, nullptr) == FA_ERR_ALIGN);
  EXPECT(fa_fwd(q, k, v, o, reinterpret_cast<float*>(reinterpret_cast<char*>(lse) + 2), B, H, N, d, sc, nullptr) ==
         FA_ERR_ALIGN);
  EXPECT(fa_fwd(q, k, v, q, lse, B, H, N, d, sc, nullptr) == FA_ERR_ALIAS);             // o is q
  EXPECT(fa_fwd(q, k, v, k + 1024, lse, B, H, N, d, sc, nullptr) == FA_ERR_ALIAS);      // o inside k
  EXPECT(fa_fwd(q, k, v, o, reinterpret_cast<float*>(o + 64), B, H, N, d, sc, nullptr) == FA_ERR_ALIAS);
  EXPECT(fa_fwd(q, k, v, o, reinterpret_cast<float*>(v), B, H, N, d, sc, nullptr) == FA_ERR_ALIAS);
  EXPECT(fa_fwd(q, k, v, o, lse, 65536, 65536, 65536, d, sc, nullptr) == FA_ERR_OVERFLOW);
  const int imax = std::numeric_limits<int>::max();
  EXPECT(fa_fwd(q, k, v, o, lse, imax, imax, imax, 128, sc, nullptr) == FA_ERR_OVERFLOW);
  EXPECT(fa_fwd(q, k, v, o, lse, 1, 1 << 16, 1 << 24, 128, sc, nullptr) == FA_ERR_OVERFLOW);  // grid > 2^31
  EXPECT(g_launches == before);

  // Q, K and V may share memory; an empty problem is a no-op even with null pointers.
  EXPECT(fa_check_args(q, q, q, o, lse, B, H, N, d, sc, 0, nullptr, 0) == FA_OK);
  EXPECT(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, H, N, d, sc, nullptr) == FA_OK);
  EXPECT(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, B, H, 0, d, sc, nullptr) == FA_OK);
  EXPECT(g_launches == before);
  // scale = 0 is allowed (the uniform average).
  EXPECT(fa_check_args(q, k, v, o, lse, B, H, N, d, 0.0f, 0, nullptr, 0) == FA_OK);

  // Overlap arithmetic at the top of the address space: adjacent ranges that end at
  // the last byte do not overlap; ranges that share it do.
  const uintptr_t top = std::numeric_limits<uintptr_t>::max() - tb + 1;  // o ends at the last byte
  const void* o_top = reinterpret_cast<const void*>(top & ~uintptr_t(255));
  EXPECT(fa_check_args(q, k, v, o_top, lse, B, H, N, d, sc, 0, nullptr, 0) == FA_OK);
  const void* q_top = reinterpret_cast<const void*>((top & ~uintptr_t(255)) + 256);
  EXPECT(fa_check_args(q_top, k, v, o_top, lse, B, H, N, d, sc, 0, nullptr, 0) == FA_ERR_ALIAS);

  // Unfused: workspace size, and each workspace error.
  const size_t need = fa_unfused_workspace_bytes(B, H, N);
  EXPECT(need == (size_t)6 * B * H * N * 128);  // N = 100 padded to 128 columns; already a multiple of 256
  EXPECT(fa_unfused_workspace_bytes(1, 1, 1) == 512);  // 6 * 64 = 384, rounded up to 256
  EXPECT(fa_unfused_workspace_bytes(0, 5, 5) == 0);
  EXPECT(fa_unfused_workspace_bytes(-1, 5, 5) == 0);
  EXPECT(fa_unfused_workspace_bytes(imax, imax, imax) == 0);
  char* ws = static_cast<char*>(std::aligned_alloc(256, need + 256));
  EXPECT(fa_unfused_fwd(q, k, v, o, lse, B, H, N, d, sc, ws, need, nullptr) == FA_OK && g_launches == before + 1);
  EXPECT(fa_unfused_fwd(q, k, v, o, lse, B, H, N, d, sc, nullptr, need, nullptr) == FA_ERR_WORKSPACE);
  EXPECT(fa_unfused_fwd(q, k, v, o, lse, B, H, N, d, sc, ws, need - 1, nullptr) == FA_ERR_WORKSPACE);
  EXPECT(fa_unfused_fwd(q, k, v, o, lse, B, H, N, d, sc, ws + 8, need, nullptr) == FA_ERR_WORKSPACE);
  EXPECT(fa_unfused_fwd(q, k, v, o, lse, B, H, N, d, sc, q, need, nullptr) == FA_ERR_WORKSPACE);
  EXPECT(g_launches == before + 1);

  // Explicit query-tile height: 128 and 256 launch with that height; any other
  // height, and the usual argument errors, return before a launch. fa_fwd launches
  // the selector's height.
  {
    const int before_blk = g_launches;
    EXPECT(fa_fwd_blocks(q, k, v, o, lse, B, H, N, d, sc, 128, nullptr) == FA_OK && g_last_br == 128);
    EXPECT(fa_fwd_blocks(q, k, v, o, lse, B, H, N, d, sc, 256, nullptr) == FA_OK && g_last_br == 256);
    EXPECT(fa_fwd_blocks(q, k, v, o, lse, B, H, N, d, sc, 64, nullptr) == FA_ERR_SHAPE);
    EXPECT(fa_fwd_blocks(q, k, v, o, lse, B, H, N, d, sc, 0, nullptr) == FA_ERR_SHAPE);
    EXPECT(fa_fwd_blocks(q, k, v, q, lse, B, H, N, d, sc, 128, nullptr) == FA_ERR_ALIAS);
    EXPECT(fa_fwd_blocks(q, k, v, o, lse, B, H, N, 96, sc, 128, nullptr) == FA_ERR_HEADDIM);
    EXPECT(fa_fwd_blocks(nullptr, nullptr, nullptr, nullptr, nullptr, 0, H, N, d, sc, 128, nullptr) == FA_OK);
    EXPECT(g_launches == before_blk + 2);
    int sbr = 0, sbc = 0, snw = 0;
    EXPECT(fa_select_blocks(d, N, B, H, &sbr, &sbc, &snw) == FA_OK);
    EXPECT(fa_fwd(q, k, v, o, lse, B, H, N, d, sc, nullptr) == FA_OK && g_last_br == sbr);
    EXPECT(g_launches == before_blk + 3);
  }

  // Decode: q/o hold Nq = 4 rows, k/v the N = 100 keys of each head.
  {
    g_device = 1;
    const int nq = 4;
    int splits = 0, chunk = 0;
    size_t dneed = 0;
    EXPECT(fa_decode_plan(B, H, nq, N, d, &splits, &chunk, &dneed) == FA_OK);
    EXPECT(splits == 1 && chunk == N && dneed == ((size_t)B * H * nq * (d + 1) * 4 + 255) / 256 * 256);
    EXPECT(fa_decode_plan(B, H, nq, N, d, nullptr, nullptr, nullptr) == FA_OK);
    int s2 = 0, c2 = 0;
    size_t w2 = 1;
    EXPECT(fa_decode_plan(B, H, 17, N, d, &s2, &c2, &w2) == FA_ERR_SHAPE && w2 == 0);
    w2 = 1;
    EXPECT(fa_decode_plan(imax, imax, 16, 1 << 30, d, &s2, &c2, &w2) == FA_ERR_OVERFLOW && w2 == 0);
    char* dws = static_cast<char*>(std::aligned_alloc(256, dneed));
    const int before_dec = g_launches;
    EXPECT(fa_decode_fwd(q, k, v, o, lse, B, H, nq, N, d, sc, dws, dneed, nullptr) == FA_OK &&
           g_launches == before_dec + 1);
    EXPECT(fa_decode_fwd(q, k, v, o, lse, B, H, nq, N, d, sc, dws, dneed - 1, nullptr) == FA_ERR_WORKSPACE);
    EXPECT(fa_decode_fwd(q, k, v, o, lse, B, H, 0, N, d, sc, nullptr, 0, nullptr) == FA_OK);
    EXPECT(fa_decode_fwd(q, k, v, o, lse, B, H, nq, 0, d, sc, dws, dneed, nullptr) == FA_ERR_SHAPE);
    EXPECT(fa_decode_fwd(q, k, v, k, lse, B, H, nq, N, d, sc, dws, dneed, nullptr) == FA_ERR_ALIAS);
    EXPECT(fa_decode_check_args(q, k, v, o, lse, B, H, nq, N, d, sc, v, dneed) == FA_ERR_WORKSPACE);
    g_device = 0;
    EXPECT(fa_decode_fwd(q, k, v, o, lse, B, H, nq, N, d, sc, dws, dneed, nullptr) == FA_ERR_DEVICE);
    EXPECT(g_launches == before_dec + 1);
    std::free(dws);
  }

  // Backward: q k v o lse dO as inputs, dq dk dv outputs (reusing the buffers above
  // for inputs and fresh ones for outputs), workspace 8*B*H*N bytes.
  {
    g_device = 1;
    char* dq = static_cast<char*>(std::aligned_alloc(256, tb));
    char* dk = static_cast<char*>(std::aligned_alloc(256, tb));
    char* dv = static_cast<char*>(std::aligned_alloc(256, tb));
    const size_t bneed = fa_bwd_workspace_bytes(B, H, N);
    EXPECT(bneed == ((size_t)8 * B * H * N + 255) / 256 * 256);
    char* bws = static_cast<char*>(std::aligned_alloc(256, bneed));
    const int before_b = g_launches;
    EXPECT(fa_bwd(q, k, v, o, lse, o, dq, dk, dv, B, H, N, d, sc, bws, bneed, nullptr) == FA_OK &&
           g_launches == before_b + 1);
    EXPECT(fa_bwd(q, k, v, o, lse, o, dq, dk, dq, B, H, N, d, sc, bws, bneed, nullptr) == FA_ERR_ALIAS);
    EXPECT(fa_bwd(q, k, v, o, lse, o, dq, dk, q, B, H, N, d, sc, bws, bneed, nullptr) == FA_ERR_ALIAS);
    EXPECT(fa_bwd(q, k, v, o, lse, nullptr, dq, dk, dv, B, H, N, d, sc, bws, bneed, nullptr) == FA_ERR_NULL);
    EXPECT(fa_bwd(q, k, v, o, lse, o, dq, dk, dv, B, H, N, d, sc, bws, bneed - 1, nullptr) == FA_ERR_WORKSPACE);
    EXPECT(fa_bwd(q, k, v, o, lse, o, dq, dk, dv, B, H, N, d, sc, dv, bneed, nullptr) == FA_ERR_WORKSPACE);
    EXPECT(fa_bwd(q, k, v, o, lse, o, dq, dk, dv, B, H, N, 96, sc, bws, bneed, nullptr) == FA_ERR_HEADDIM);
    EXPECT(g_launches == before_b + 1);
    std::free(bws);
    std::free(dq);
    std::free(dk);
    std::free(dv);
  }

  // Selector and strings.
  int br = 0, bc = 0, nw = 0;
  EXPECT(fa_select_blocks(128, 8192, 1, 32, &br, &bc, &nw) == FA_OK && br == 256 && bc == 64 && nw == 4);
  EXPECT(fa_select_blocks(64, 1024, 4, 16, &br, &bc, &nw) == FA_OK && br == 128 && bc == 64 && nw == 4);
  EXPECT(fa_select_blocks(128, 8192, 1, 8, &br, &bc, &nw) == FA_OK && br == 256);   // 256 tiles: one full round
  EXPECT(fa_select_blocks(128, 8192, 1, 4, &br, &bc, &nw) == FA_OK && br == 128);   // 128 tiles: half the CUs
  EXPECT(fa_select_blocks(128, 30001, 1, 8, &br, &bc, &nw) == FA_OK && br == 256);
  EXPECT(fa_select_blocks(128, 8192, -1, 8, &br, &bc, &nw) == FA_ERR_SHAPE);
  EXPECT(fa_select_blocks(80, 1024, 4, 16, &br, &bc, &nw) == FA_ERR_HEADDIM);
  EXPECT(fa_select_blocks(64, 1024, 4, 16, nullptr, &bc, &nw) == FA_ERR_NULL);
  for (int s = FA_ERR_DEVICE; s <= FA_OK; ++s) {
    const char* str = fa_status_string(s);
    EXPECT(str != nullptr && std::strlen(str) > 0 && std::strcmp(str, "unknown status") != 0);
  }
  EXPECT(std::strcmp(fa_status_string(12345), "unknown status") == 0);
  EXPECT(fa_version() >= 10000);

  // The allocation-free decode: argument errors and a shape whose partial results do
  // not fit the fixed scratch array return before any launch or scratch lookup.
  {
    const int before_nl = g_launches;
    EXPECT(fa_decode_fwd_noalloc(q, k, v, o, lse, B, H, 17, N, d, sc, nullptr) == FA_ERR_SHAPE);
    EXPECT(fa_decode_fwd_noalloc(q, k, v, q, lse, B, H, 4, N, d, sc, nullptr) == FA_ERR_ALIAS);
    EXPECT(fa_decode_fwd_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, 0, H, 4, N, d, sc, nullptr) == FA_OK);
    // 64*64 heads of 16 rows, one key chunk each: 16.9 M floats of partials > 32 MiB
    EXPECT(fa_decode_fwd_noalloc(q, k, v, o, lse, 64, 64, 16, 4096, 128, sc, nullptr) == FA_ERR_SCRATCH ||
           fa_decode_fwd_noalloc(q, k, v, o, lse, 64, 64, 16, 4096, 128, sc, nullptr) == FA_ERR_ALIAS);
    EXPECT(g_launches == before_nl && fa::g_scratch_lookups == 0);
    // a valid small call looks the array up and launches once
    EXPECT(fa_decode_fwd_noalloc(q, k, v, o, lse, B, H, 4, N, d, sc, nullptr) == FA_OK);
    EXPECT(g_launches == before_nl + 1 && fa::g_scratch_lookups == 1);
  }

  std::free(ws);
  std::free(q);
  std::free(k);
  std::free(v);
  std::free(o);
  std::free(lse);
  if (g_failures == 0) std::printf("check_args: all passed\n");
  return g_failures == 0 ? 0 : 1;
}
