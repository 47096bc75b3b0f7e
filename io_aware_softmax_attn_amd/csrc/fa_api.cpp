// C ABI of libfa.so: argument validation, dispatch and status strings.
// Plain host C++ (no HIP headers); the HIP work happens behind fa_internal.h.
#include "../../include/fa.h"

#include <cmath>
#include <cstdint>
#include <limits>

#include "fa_internal.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

// Whether [a, a+na) and [b, b+nb) share a byte. Written with differences only, so
// ranges near the top of the address space cannot wrap the comparison.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa <= pb ? pb - pa < na : pa - pb < nb;
}

bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
  if (a != 0 && b > std::numeric_limits<uint64_t>::max() / a) return false;
  *out = a * b;
  return true;
}

}  // namespace

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H and N must be >= 0 (decode: 1 <= Nq <= 16 and 1 <= Nk <= 2^30)";
    case FA_ERR_HEADDIM: return "head dimension d must be 64 or 128";
    case FA_ERR_ALIGN: return "q, k, v, o and workspace must be 16-byte aligned, lse 4-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_ALIAS: return "o or lse overlaps an input, or each other";
    case FA_ERR_OVERFLOW: return "problem size overflows 64-bit byte counts or the launch grid";
    case FA_ERR_WORKSPACE: return "workspace is missing, too small, misaligned or overlaps a tensor";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_DEVICE: return "current device is not gfx950 (MI355X)";
    case FA_ERR_SCRATCH: return "the problem needs more than FA_DECODE_SCRATCH_BYTES of the library's fixed scratch buffer";
    default: return "unknown status";
  }
}

size_t fa_unfused_workspace_bytes(int B, int H, int N) {
  if (B < 0 || H < 0 || N < 0) return 0;
  // S (fp32) and P (bf16) rows are padded to a multiple of 64 columns.
  const uint64_t ns = ((uint64_t)N + 63) / 64 * 64;
  uint64_t rows, sq, bytes;
  if (!mul_ok((uint64_t)B * (uint64_t)H, (uint64_t)N, &rows)) return 0;
  if (!mul_ok(rows, ns, &sq)) return 0;
  if (!mul_ok(sq, 6, &bytes)) return 0;
  if (bytes > std::numeric_limits<uint64_t>::max() - 255) return 0;
  bytes = (bytes + 255) & ~uint64_t(255);
  if (bytes > std::numeric_limits<size_t>::max()) return 0;
  return (size_t)bytes;
}

int fa_select_blocks(int d, int N, int B, int H, int* br, int* bc, int* nwaves) {
  if (!br || !bc || !nwaves) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  const fa::Blocks b = fa::select_blocks(d, N, B, H);
  *br = b.br;
  *bc = b.bc;
  *nwaves = b.nwaves;
  return FA_OK;
}

int fa_check_args(const void* q, const void* k, const void* v, const void* o, const void* lse,
                  int B, int H, int N, int d, float scale,
                  int need_workspace, const void* workspace, size_t workspace_bytes) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  // B, H, N < 2^31, so B*H < 2^62 and B*H*N cannot wrap once B*H < 2^33.
  if ((uint64_t)B * (uint64_t)H > (std::numeric_limits<uint64_t>::max() >> 31)) return FA_ERR_OVERFLOW;
  const uint64_t rows64 = (uint64_t)B * (uint64_t)H * (uint64_t)N;
  if (rows64 == 0) return FA_OK;  // empty problem: nothing is touched
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  uint64_t elems, tbytes, lbytes;
  if (!mul_ok(rows64, (uint64_t)d, &elems) || !mul_ok(elems, 2, &tbytes) || !mul_ok(rows64, 4, &lbytes))
    return FA_ERR_OVERFLOW;
  // Launch grid: one workgroup per (b, h, query tile); the narrowest tile has 128 rows.
  const uint64_t tiles = ((uint64_t)N + 127) / 128;
  if ((uint64_t)B * (uint64_t)H * tiles > (uint64_t)std::numeric_limits<int32_t>::max()) return FA_ERR_OVERFLOW;
  auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4))
    return FA_ERR_ALIGN;
  const size_t tb = (size_t)tbytes, lb = (size_t)lbytes;
  if (overlaps(o, tb, q, tb) || overlaps(o, tb, k, tb) || overlaps(o, tb, v, tb) || overlaps(lse, lb, q, tb) ||
      overlaps(lse, lb, k, tb) || overlaps(lse, lb, v, tb) || overlaps(lse, lb, o, tb))
    return FA_ERR_ALIAS;
  if (need_workspace) {
    const size_t need = fa_unfused_workspace_bytes(B, H, N);
    if (need == 0) return FA_ERR_OVERFLOW;
    if (!workspace || workspace_bytes < need || misaligned(workspace, 16)) return FA_ERR_WORKSPACE;
    if (overlaps(workspace, need, q, tb) || overlaps(workspace, need, k, tb) || overlaps(workspace, need, v, tb) ||
        overlaps(workspace, need, o, tb) || overlaps(workspace, need, lse, lb))
      return FA_ERR_WORKSPACE;
  }
  return FA_OK;
}

int fa_decode_plan(int B, int H, int Nq, int Nk, int d, int* splits, int* chunk, size_t* workspace_bytes) {
  if (workspace_bytes) *workspace_bytes = 0;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || Nq > FA_DECODE_MAX_NQ || Nk > FA_DECODE_MAX_NK) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if ((uint64_t)B * (uint64_t)H > (std::numeric_limits<uint64_t>::max() >> 31)) return FA_ERR_OVERFLOW;
  const fa::DecodePlan p = fa::decode_plan(B, H, Nq, Nk, d);
  uint64_t groups, rows, floats, bytes;
  if (!mul_ok((uint64_t)B * (uint64_t)H, (uint64_t)p.splits, &groups) || !mul_ok(groups, (uint64_t)Nq, &rows) ||
      !mul_ok(rows, (uint64_t)d + 1, &floats) || !mul_ok(floats, 4, &bytes) ||
      bytes > std::numeric_limits<uint64_t>::max() - 255)
    return FA_ERR_OVERFLOW;
  bytes = (bytes + 255) & ~uint64_t(255);
  if (bytes > std::numeric_limits<size_t>::max()) return FA_ERR_OVERFLOW;
  if (splits) *splits = p.splits;
  if (chunk) *chunk = p.chunk;
  if (workspace_bytes) *workspace_bytes = (size_t)bytes;
  return FA_OK;
}

}  // extern "C"

namespace {

// Every check of fa_decode_check_args except the workspace's: shapes, pointers,
// alignment and overlaps. *need receives the workspace bytes (0 for an empty
// problem).
int decode_check_tensors(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int H,
                         int Nq, int Nk, int d, float scale, size_t* need_out, size_t* qs_out, size_t* ks_out,
                         size_t* ls_out) {
  *need_out = 0;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if ((uint64_t)B * (uint64_t)H > (std::numeric_limits<uint64_t>::max() >> 31)) return FA_ERR_OVERFLOW;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  const uint64_t rows64 = bh * (uint64_t)Nq;
  if (rows64 == 0) return FA_OK;  // empty problem: nothing is touched
  if (Nq > FA_DECODE_MAX_NQ || Nk < 1 || Nk > FA_DECODE_MAX_NK) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int splits = 0;
  size_t need = 0;
  const int pst = fa_decode_plan(B, H, Nq, Nk, d, &splits, nullptr, &need);
  if (pst != FA_OK) return pst;
  uint64_t qb, kb, lb, groups;
  if (!mul_ok(rows64 * (uint64_t)d, 2, &qb) || !mul_ok(bh * (uint64_t)Nk, (uint64_t)d * 2, &kb) ||
      !mul_ok(rows64, 4, &lb) || !mul_ok(bh, (uint64_t)splits, &groups))
    return FA_ERR_OVERFLOW;
  // Launch grids: B*H*splits split workgroups, B*H*Nq merge rows.
  if (groups > (uint64_t)std::numeric_limits<int32_t>::max() || rows64 > (uint64_t)std::numeric_limits<int32_t>::max())
    return FA_ERR_OVERFLOW;
  auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4))
    return FA_ERR_ALIGN;
  const size_t qs = (size_t)qb, ks = (size_t)kb, ls = (size_t)lb;
  if (overlaps(o, qs, q, qs) || overlaps(o, qs, k, ks) || overlaps(o, qs, v, ks) || overlaps(lse, ls, q, qs) ||
      overlaps(lse, ls, k, ks) || overlaps(lse, ls, v, ks) || overlaps(lse, ls, o, qs))
    return FA_ERR_ALIAS;
  *need_out = need;
  *qs_out = qs;
  *ks_out = ks;
  *ls_out = ls;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_decode_check_args(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int H,
                         int Nq, int Nk, int d, float scale, const void* workspace, size_t workspace_bytes) {
  size_t need = 0, qs = 0, ks = 0, ls = 0;
  const int st = decode_check_tensors(q, k, v, o, lse, B, H, Nq, Nk, d, scale, &need, &qs, &ks, &ls);
  if (st != FA_OK || need == 0) return st;
  auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
  if (!workspace || workspace_bytes < need || misaligned(workspace, 16)) return FA_ERR_WORKSPACE;
  if (overlaps(workspace, need, q, qs) || overlaps(workspace, need, k, ks) || overlaps(workspace, need, v, ks) ||
      overlaps(workspace, need, o, qs) || overlaps(workspace, need, lse, ls))
    return FA_ERR_WORKSPACE;
  return FA_OK;
}

int fa_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                          int Nk, int d, float scale, void* stream) {
  size_t need = 0, qs = 0, ks = 0, ls = 0;
  const int st = decode_check_tensors(q, k, v, o, lse, B, H, Nq, Nk, d, scale, &need, &qs, &ks, &ls);
  if (st != FA_OK || need == 0) return st;  // need == 0: empty problem, a no-op
  if (need > (size_t)FA_DECODE_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  const int dev = fa::device_is_gfx950();
  if (dev < 0) return dev;
  if (dev == 0) return FA_ERR_DEVICE;
  void* buf = nullptr;  // device address of the fixed scratch array on this device
  const int sst = fa::decode_scratch(&buf);
  if (sst != FA_OK) return sst;
  return fa::launch_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, buf, stream);
}

int fa_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int d,
                  float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = fa_decode_check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)Nq == 0) return FA_OK;
  const int dev = fa::device_is_gfx950();
  if (dev < 0) return dev;
  if (dev == 0) return FA_ERR_DEVICE;
  return fa::launch_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, workspace, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, float scale,
           void* stream) {
  const int st = fa_check_args(q, k, v, o, lse, B, H, N, d, scale, 0, nullptr, 0);
  if (st != FA_OK) return st;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)N == 0) return FA_OK;
  const int dev = fa::device_is_gfx950();
  if (dev < 0) return dev;
  if (dev == 0) return FA_ERR_DEVICE;
  return fa::launch_fused(q, k, v, o, lse, B, H, N, d, scale, fa::select_blocks(d, N, B, H), stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 0 || H < 0 || N < 0) return 0;
  uint64_t rows, bytes;
  if (!mul_ok((uint64_t)B * (uint64_t)H, (uint64_t)N, &rows) || !mul_ok(rows, 8, &bytes) ||
      bytes > std::numeric_limits<uint64_t>::max() - 255)
    return 0;
  bytes = (bytes + 255) & ~uint64_t(255);
  if (bytes > std::numeric_limits<size_t>::max()) return 0;
  return (size_t)bytes;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
           void* dk, void* dv, int B, int H, int N, int d, float scale, void* workspace, size_t workspace_bytes,
           void* stream) {
  // q, k, v, o, lse as the forward's arguments (o and lse are inputs here).
  const int st = fa_check_args(q, k, v, o, lse, B, H, N, d, scale, 0, nullptr, 0);
  if (st != FA_OK) return st;
  const uint64_t rows64 = (uint64_t)B * (uint64_t)H * (uint64_t)N;
  if (rows64 == 0) return FA_OK;
  if (!dO || !dq || !dk || !dv) return FA_ERR_NULL;
  // Launch grid: one workgroup per (b, h, 128 rows).
  if ((uint64_t)B * (uint64_t)H * (((uint64_t)N + 127) / 128) > (uint64_t)std::numeric_limits<int32_t>::max())
    return FA_ERR_OVERFLOW;
  auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
  if (misaligned(dO, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16)) return FA_ERR_ALIGN;
  const size_t tb = (size_t)(rows64 * (uint64_t)d * 2), lb = (size_t)(rows64 * 4);
  const void* ins[6] = {q, k, v, o, lse, dO};
  const size_t in_bytes[6] = {tb, tb, tb, tb, lb, tb};
  void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], tb, ins[j], in_bytes[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], tb, outs[j], tb)) return FA_ERR_ALIAS;
  }
  const size_t need = fa_bwd_workspace_bytes(B, H, N);
  if (need == 0) return FA_ERR_OVERFLOW;
  if (!workspace || workspace_bytes < need || misaligned(workspace, 16)) return FA_ERR_WORKSPACE;
  for (int j = 0; j < 6; ++j)
    if (overlaps(workspace, need, ins[j], in_bytes[j])) return FA_ERR_WORKSPACE;
  for (int i = 0; i < 3; ++i)
    if (overlaps(workspace, need, outs[i], tb)) return FA_ERR_WORKSPACE;
  const int dev = fa::device_is_gfx950();
  if (dev < 0) return dev;
  if (dev == 0) return FA_ERR_DEVICE;
  return fa::launch_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, workspace, stream);
}

int fa_fwd_tile_order(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                      float scale, int order, void* stream) {
  if (order < 0 || order > 2) return FA_ERR_SHAPE;
  const int st = fa_check_args(q, k, v, o, lse, B, H, N, d, scale, 0, nullptr, 0);
  if (st != FA_OK) return st;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)N == 0) return FA_OK;
  const int dev = fa::device_is_gfx950();
  if (dev < 0) return dev;
  if (dev == 0) return FA_ERR_DEVICE;
  return fa::launch_fused(q, k, v, o, lse, B, H, N, d, scale, fa::select_blocks(d, N, B, H), stream, order);
}

int fa_fwd_blocks(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                  float scale, int br, void* stream) {
  if (br != 128 && br != 256) return FA_ERR_SHAPE;
  const int st = fa_check_args(q, k, v, o, lse, B, H, N, d, scale, 0, nullptr, 0);
  if (st != FA_OK) return st;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)N == 0) return FA_OK;
  const int dev = fa::device_is_gfx950();
  if (dev < 0) return dev;
  if (dev == 0) return FA_ERR_DEVICE;
  fa::Blocks blk = fa::select_blocks(d, N, B, H);
  blk.br = br;
  return fa::launch_fused(q, k, v, o, lse, B, H, N, d, scale, blk, stream);
}

int fa_unfused_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = fa_check_args(q, k, v, o, lse, B, H, N, d, scale, 1, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)N == 0) return FA_OK;
  const int dev = fa::device_is_gfx950();
  if (dev < 0) return dev;
  if (dev == 0) return FA_ERR_DEVICE;
  return fa::launch_unfused(q, k, v, o, lse, B, H, N, d, scale, workspace, stream);
}

}  // extern "C"
