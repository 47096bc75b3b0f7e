/*
 * fa.h - C ABI of the MI355X (gfx950) attention-forward library, libfa.so.
 *
 * The library computes the exact attention forward of the FlashAttention pages:
 *     O   = softmax(scale * Q K^T) V          (row-wise softmax over the keys)
 *     LSE = per query row, ln sum_j exp(scale * q_i . k_j)
 * in one fused kernel that never stores the N x N scores or probabilities
 * ("Flash Attention (FA1)", sections "Tiling in FlashAttention" and
 * "Online Softmax in FlashAttention"; "01 · 注意力为什么是 IO 瓶颈", section 4:
 * read Q, K, V once, write O and LSE once). It also ships the textbook
 * three-kernel computation (same page, section 3 table: S = QK^T to memory,
 * P = softmax(S) to memory, O = PV) as a traffic baseline, and the block-size
 * selector ("01 ·" page, section 7: tile sizes are chosen against on-chip
 * memory capacity).
 *
 * Conventions for every entry point:
 *   - Tensors are dense, contiguous, row-major [B, H, N, d] (Q, K, V, O; bf16)
 *     and [B, H, N] (LSE; fp32), in device memory the caller allocated and owns.
 *     The library allocates nothing on the fused path and keeps no pointer after
 *     a call returns.
 *   - d (head dimension) must be 64 or 128. B, H, N >= 0; when B*H*N == 0 the
 *     call is a no-op that returns FA_OK without touching any pointer.
 *   - scale must be finite, of either sign (the pages' scale is 1/sqrt(d) > 0; 0
 *     gives the uniform average; a negative scale is the softmax of the negated
 *     scores, which the running max handles like any other).
 *   - Q, K, V, O must be 16-byte aligned; LSE 4-byte aligned. Q, K and V may
 *     share memory; O and LSE must not overlap any input or each other.
 *   - Work is launched on the calling thread's current HIP device; the tensors
 *     and the stream must belong to it.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream). Calls
 *     are asynchronous: they return after enqueueing the work; faults during
 *     execution surface at the caller's next synchronisation on that stream.
 *   - Argument errors are detected before any HIP call and return a negative
 *     fa_status; nothing is enqueued then. A launch error returns FA_ERR_HIP.
 *   - The fused result is bitwise deterministic for a given device and shape
 *     (no atomics, fixed reduction order).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,     /* B, H or N negative; decode: Nq or Nk out of range */
  FA_ERR_HEADDIM = -3,   /* d not in {64, 128} */
  FA_ERR_ALIGN = -4,     /* a pointer is not aligned as stated above */
  FA_ERR_SCALE = -5,     /* scale not finite */
  FA_ERR_ALIAS = -6,     /* O or LSE overlaps an input or each other */
  FA_ERR_OVERFLOW = -7,  /* sizes overflow 64-bit byte counts or the launch grid */
  FA_ERR_WORKSPACE = -8, /* workspace missing, too small, misaligned or overlapping */
  FA_ERR_HIP = -9,       /* the HIP runtime reported an error */
  FA_ERR_DEVICE = -10,   /* the current device is not gfx950 */
  FA_ERR_SCRATCH = -11   /* the problem needs more than the library's fixed scratch buffer */
} fa_status;

/*
 * Fused attention forward. q, k, v, o: bf16 [B,H,N,d]; lse: fp32 [B,H,N].
 * Per row i of each (b, h): o[i] = sum_j p_ij v[j] / sum_j p_ij with
 * p_ij = exp(s_ij - max_j s_ij), s_ij = scale * q[i].k[j]; lse[i] = ln sum_j exp(s_ij).
 * One kernel launch: Q is tiled by rows, K/V stream through on-chip memory in
 * column tiles, and the online softmax (running max, running sum, rescaled
 * accumulator; "Flash Attention (FA1)", derivation steps 1-5) keeps S and P on
 * chip. O is rounded to bf16 (nearest-even) once, at the end. The query-tile
 * height is the one fa_select_blocks returns for the shape.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, void* stream);

/*
 * fa_fwd with an explicit order in which workgroups take the (b, h, query tile)
 * tiles, for measuring how the reuse of K/V across a head's query tiles in the
 * on-chip caches sets the memory traffic. The pages count the traffic of the
 * tiled method as K and V re-read once per query tile, about N^2 d^2 / M element
 * accesses for on-chip memory M ("01 · 注意力为什么是 IO 瓶颈", section 7), and
 * O(N d) when those re-reads are served on chip (same page, section 4).
 *   order 0: fa_fwd's order: each XCD takes a contiguous range of tiles, so a
 *            head's query tiles share that XCD's L2;
 *   order 1: dispatch order: a head's consecutive tiles go to all 8 XCDs;
 *   order 2: query-tile-major: consecutive workgroups belong to different heads,
 *            so a head's tiles are spread over XCDs and time.
 * Results are bitwise identical for every order. Returns FA_ERR_SHAPE for an
 * order outside 0..2; otherwise as fa_fwd.
 */
int fa_fwd_tile_order(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int order, void* stream);

/*
 * fa_fwd with an explicit query-tile height br (rows of Q per workgroup): 256 or
 * 128, the two compiled shapes (4 waves of 64 or 32 rows, 64-key K/V tiles). The
 * pages size the query tile against on-chip memory ("01 · 注意力为什么是 IO 瓶颈",
 * section 7) and count the K/V traffic as one pass per query tile (same section);
 * this entry point lets a caller compare the two heights. Results for a given
 * br are bitwise deterministic; the two heights may differ in the last bits, as
 * a wave decides when to move its softmax reference over its own rows. Returns
 * FA_ERR_SHAPE for any other br; otherwise as fa_fwd.
 */
int fa_fwd_blocks(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, float scale, int br, void* stream);

/*
 * The textbook three-step forward ("01 · 注意力为什么是 IO 瓶颈", section 3
 * table and section 5): kernel 1 writes S = scale*QK^T (fp32, [B,H,N,Ns]) to the
 * workspace, kernel 2 reads S and writes P = softmax(S) (bf16, [B,H,N,Ns]) and
 * LSE, kernel 3 reads P and V and writes O. Same argument rules as fa_fwd, plus
 * a caller-owned device workspace of at least fa_unfused_workspace_bytes(B,H,N)
 * bytes, 16-byte aligned, not overlapping any tensor argument.
 */
int fa_unfused_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_unfused_fwd needs: 6*B*H*N*Ns with Ns = N rounded up to a
 * multiple of 64 (fp32 S + bf16 P, rows padded), rounded up to 256; 0 if the
 * product overflows size_t. */
size_t fa_unfused_workspace_bytes(int B, int H, int N);

/*
 * Block-size selector: the (query rows per workgroup, keys per tile, waves per
 * workgroup) the fused kernel uses for this shape ("01 ·" page, section 7: tiles
 * are sized against on-chip memory; kp-015 page, "常见误区": the gain depends on
 * the number of compute units). br is 256 or 128, bc is 64, nwaves is 4; the
 * choice depends on the shape only (d, N, B*H against the 256 compute units of
 * the part), never on the device the call runs on, so results stay a function
 * of the shape. Writes *br, *bc, *nwaves; returns FA_OK, FA_ERR_NULL,
 * FA_ERR_SHAPE (B, H or N negative) or FA_ERR_HEADDIM.
 */
int fa_select_blocks(int d, int N, int B, int H, int* br, int* bc, int* nwaves);

/*
 * Argument validation shared by fa_fwd and fa_unfused_fwd, exposed so callers
 * can check arguments without a GPU. workspace may be NULL for the fused path
 * (need_workspace = 0). Pure host code: makes no HIP call.
 */
int fa_check_args(const void* q, const void* k, const void* v, const void* o, const void* lse,
                  int B, int H, int N, int d, float scale,
                  int need_workspace, const void* workspace, size_t workspace_bytes);

/*
 * Decode-shaped forward: Nq query rows per head (1 <= Nq <= FA_DECODE_MAX_NQ)
 * against Nk keys (1 <= Nk <= FA_DECODE_MAX_NK), the workload the KP page
 * contrasts with prefill ("FlashAttention：IO 感知的精确注意力", sections 常见误区
 * and 自测题: decode is limited by memory traffic). q, o: bf16 [B,H,Nq,d];
 * k, v: bf16 [B,H,Nk,d]; lse: fp32 [B,H,Nq]. Same definition as fa_fwd, with
 * j running over the Nk keys: o[i] = sum_j p_ij v[j] / sum_j p_ij and
 * lse[i] = ln sum_j exp(s_ij). Same conventions as above (d in {64, 128},
 * alignment, no overlap of o and lse with anything, asynchronous on stream),
 * plus a caller-owned device workspace of at least the bytes fa_decode_plan
 * reports, 16-byte aligned and overlapping no tensor argument.
 *
 * Two kernels: the first splits each head's keys into chunks, one workgroup per
 * chunk, and writes each chunk's normalised partial O and its LSE (fp32) to the
 * workspace; the second merges the partials of each row with the FA1 page's
 * update (derivation steps 2 and 4-5) applied to whole chunks. Scores are fp32
 * (bf16 products accumulate exactly in fp32); probabilities keep about 16 bits
 * (fp32 for one query row; as a bf16 pair, value and remainder, on the matrix
 * cores for 2 to 16 rows); O is rounded to bf16 (nearest-even) once, at the end.
 * When B*H*Nq == 0 the call is a no-op. Deterministic for a given shape: the
 * split depends on the shape only.
 */
#define FA_DECODE_MAX_NQ 16
#define FA_DECODE_MAX_NK (1 << 30)
int fa_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, float scale,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * The key split fa_decode_fwd uses for this shape: *splits chunks of *chunk keys
 * per (b, h) (the last chunk may be shorter), and the workspace it needs,
 * B*H*splits*Nq*(d+1)*4 bytes rounded up to 256 (partial O, then partial LSE).
 * Any output pointer may be NULL. Returns FA_OK, FA_ERR_SHAPE, FA_ERR_HEADDIM or
 * FA_ERR_OVERFLOW (then *workspace_bytes is 0). Pure host code.
 */
int fa_decode_plan(int B, int H, int Nq, int Nk, int d, int* splits, int* chunk, size_t* workspace_bytes);

/*
 * fa_decode_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * kernels, split and results as fa_decode_fwd (bit for bit), but the partial
 * results of the key split go to a fixed device array of FA_DECODE_SCRATCH_BYTES
 * inside the library instead of a caller workspace; the array exists once per GPU
 * and is held until the process ends. The call allocates nothing, frees nothing
 * and issues no memset (the split writes every partial it reads back). The first
 * call on a device looks the array's address up for that device.
 *
 * Every call on one GPU shares that GPU's array: calls ordered on one stream are
 * safe, but calls that can overlap in time on one GPU (other streams or threads
 * without ordering between them) race on it and give wrong results. Returns
 * FA_ERR_SCRATCH, before any HIP call, when the shape needs more than
 * FA_DECODE_SCRATCH_BYTES (the workspace_bytes of fa_decode_plan); otherwise as
 * fa_decode_fwd.
 */
#define FA_DECODE_SCRATCH_BYTES (32u << 20)
int fa_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Nq, int Nk, int d, float scale, void* stream);

/* Argument validation of fa_decode_fwd, without a GPU. Pure host code. */
int fa_decode_check_args(const void* q, const void* k, const void* v, const void* o, const void* lse,
                         int B, int H, int Nq, int Nk, int d, float scale,
                         const void* workspace, size_t workspace_bytes);

/*
 * Attention backward: dq, dk, dv (bf16 [B,H,N,d]) of o = fa_fwd(q, k, v) for the
 * upstream gradient dO (bf16 [B,H,N,d]), from q, k, v and the forward's o and lse:
 *   dv = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dq = scale dS K,  dk = scale dS^T Q
 * with P = exp(scale Q K^T - lse) recomputed tile by tile and D_i = dO_i . o_i. The
 * pages keep only O and the per-row LSE from the forward and recompute P in the
 * backward ("01 · 注意力为什么是 IO 瓶颈", section 6); no N x N matrix is stored.
 * lse receives no gradient. Same conventions as fa_fwd for shapes, d, scale and
 * alignment; dq, dk and dv must not overlap each other or any input; workspace is
 * a caller-owned device buffer of at least fa_bwd_workspace_bytes(B, H, N) bytes,
 * 16-byte aligned, overlapping no tensor argument. Three kernels: per-row D and
 * lse in log2 units into the workspace; dq (one workgroup per 128 query rows); dk
 * and dv (one workgroup per 128 keys). Products are bf16 MFMA with fp32
 * accumulation; P and dS enter them rounded to bf16; outputs are rounded to bf16
 * once. Deterministic: no atomics.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_bwd needs: 8*B*H*N (fp32 D and lse in log2 units per row),
 * rounded up to 256; 0 if negative or the product overflows size_t. */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/* Utilities. Static, NUL-terminated description of a status code. */
const char* fa_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
