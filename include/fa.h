/*
 * fa.h -- exact scaled-dot-product attention, computed tile by tile with the
 * online-softmax rescale, for AMD Instinct MI355X (gfx950).  C ABI of libfa.so.
 *
 * Pages cited (title, then section):
 *   [Atlas] "FlashAttention -- IO-Aware Exact Attention" (atlas.blal.pro wiki)
 *   [ZtF]   "FlashAttention", zerotofrontier.app textbook section 12.3
 *
 * Operation ([ZtF] "The picture, a grid of tiles" and "The forward pass"):
 * for every batch b < B and head h < H independently, with S = scale * Q K^T,
 * P = softmax(S) row-wise and O = P V, plus one log-sum-exp per query row,
 * lse_r = ln sum_l exp(S_rl) ([ZtF] "What the forward pass leaves behind";
 * [Atlas] "Recomputation in the backward pass").  With `causal` set, query r
 * sees key l only when l <= r (top-left alignment, also when Tq != Tk) ([ZtF]
 * "The causal mask, and the tiles you never visit").  The backward pass returns
 * the gradients of sum(O * dO) from Q, K, V, O, dO and lse alone, recomputing
 * the probabilities tile by tile ([ZtF] "The backward pass, derived").
 *
 * Layout: every tensor is dense row-major with the head dimension fastest:
 *   Q, O, dO, dQ   [B][H][Tq][d]      K, V, dK, dV   [B][H][Tk][d]
 *   lse            [B][H][Tq] float32 (natural log)
 * Element type: FA_BF16 (bfloat16 storage, float32 accumulation) or FA_F32.
 * Supported head widths: d in {64, 128, 256}.
 *
 * Ownership: every pointer is a device pointer owned by the caller; device
 * buffers must be 16-byte aligned.  The library keeps no state between calls
 * except the per-device module handles HIP itself keeps.  Calls are
 * asynchronous on `stream` (a hipStream_t; NULL = the null stream): FA_OK means
 * every launch was accepted, and faults surface at the caller's next
 * synchronisation.  All argument checks run before any device work; on an
 * error nothing is launched and no output is touched.  NaN or Inf inputs are
 * not checked: they propagate to the outputs that depend on them (a NaN in a
 * query row reaches that row only; a NaN in a key's K row reaches only the rows
 * that see the key, since masked scores are -inf whatever their value).  A NaN
 * in a V row can also reach rows that do not see that key when its tile is
 * computed for them (a zero weight times NaN is NaN).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,       /* a required pointer is NULL                          */
  FA_ERR_SHAPE = -2,      /* B, H, Tq or Tk < 1, or a grid dimension overflows   */
  FA_ERR_HEADDIM = -3,    /* d not in {64, 128, 256}                             */
  FA_ERR_DTYPE = -4,      /* unknown dtype, or an unsupported dtype combination  */
  FA_ERR_SCALE = -5,      /* scale not finite or not > 0                         */
  FA_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than fa_bwd_workspace_bytes */
  FA_ERR_LAUNCH = -7,     /* the HIP runtime rejected a launch                   */
  FA_ERR_ALIGN = -8,      /* a device pointer is not 16-byte aligned             */
  FA_ERR_PHASE = -9,      /* unknown bits in an fa_bwd_phases mask               */
  FA_ERR_SCRATCH = -10    /* fa_bwd_noalloc: the problem needs more than the
                             library's fixed scratch (FA_NOALLOC_SCRATCH_BYTES)  */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/* Phases of the backward pass, for fa_bwd_phases. */
typedef enum {
  FA_BWD_PRE = 1,   /* row terms D = rowsum(dO * O) (and -lse log2 e) into the
                       workspace                                                    */
  FA_BWD_MAIN = 2,  /* key-block sweep: recompute P, write dK and dV                */
  FA_BWD_POST = 4,  /* query-block sweep: recompute P, write dQ                     */
  FA_BWD_ALL = 7
} fa_bwd_phase;

/*
 * Forward pass ([ZtF] "The forward pass", steps 1-3; FlashAttention-2 order:
 * one workgroup per query block, one sweep over the key/value blocks, O and
 * lse written once).
 *   Q [B][H][Tq][d], K and V [B][H][Tk][d]  (dtype)          in
 *   O [B][H][Tq][d] (out_dtype), lse [B][H][Tq] (float32)     out
 *   scale      the factor on Q K^T; the usual choice is 1/sqrt(d)
 *   causal     0 = full attention, 1 = query r sees keys l <= r
 *   out_dtype  storage type of O: the input dtype, or FA_F32 for bf16 inputs
 *              (keeps O's float32 accumulation unrounded, e.g. for a backward
 *              pass whose row terms D = dO . O must not carry bf16 rounding)
 * Returns FA_OK or an fa_status error code.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* lse,
           int B, int H, int Tq, int Tk, int d, float scale, int causal,
           int dtype, int out_dtype, void* stream);

/*
 * Bytes of device workspace fa_bwd needs, all float32 and per query row
 * ([B][H][Tq], each array rounded up to a multiple of 64 entries): the row
 * terms D_r = dO_r . O_r ([ZtF] "The backward pass, derived", Observation 2),
 * for bf16 inputs stored as -D_r next to -lse_r log2(e).  Returns 0 for
 * invalid arguments.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Tq, int Tk, int d, int dtype, int grad_dtype);

/*
 * Backward pass by recomputation ([ZtF] "The backward pass, derived"):
 *   Q, K, V, dO (dtype), O (o_dtype), lse (float32, as fa_fwd wrote it)  in
 *   dQ [B][H][Tq][d], dK and dV [B][H][Tk][d] (grad_dtype)               out
 * o_dtype and grad_dtype: the input dtype, or FA_F32 for bfloat16 inputs.
 * Two sweeps ([ZtF] "Which loop goes outside?"): one over key blocks writes dK
 * and dV, one over query blocks writes dQ; both recompute P from lse, and every
 * output is summed in a fixed order, so results repeat bit for bit.
 * workspace: device buffer of at least fa_bwd_workspace_bytes(...) bytes,
 * 16-byte aligned, owned by the caller; its contents on entry do not matter.
 * Returns FA_OK or an fa_status error code.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* lse, void* dQ, void* dK, void* dV,
           int B, int H, int Tq, int Tk, int d, float scale, int causal,
           int dtype, int o_dtype, int grad_dtype, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * The same backward pass split into its phases, for callers that schedule or
 * time them separately: `phases` is an OR of fa_bwd_phase bits, and the
 * phases it names run in the order PRE, MAIN, POST on `stream`.  Running the
 * three in that order (in one call or several, with the same arguments and
 * workspace) is exactly fa_bwd.  MAIN and POST read the row terms PRE left in
 * the workspace.  Same arguments and errors as
 * fa_bwd, plus FA_ERR_PHASE for bits outside FA_BWD_ALL; phases = 0 checks the
 * arguments and launches nothing.
 */
int fa_bwd_phases(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                  const float* lse, void* dQ, void* dK, void* dV,
                  int B, int H, int Tq, int Tk, int d, float scale, int causal,
                  int dtype, int o_dtype, int grad_dtype, void* workspace, size_t workspace_bytes,
                  int phases, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): fa_bwd with
 * no workspace argument.  Its workspace is a fixed array inside the library,
 * FA_NOALLOC_SCRATCH_BYTES long (16 MiB: fa_bwd_workspace_bytes up to that
 * size, i.e. B*H*Tq up to 2^21 query rows for bfloat16 inputs and 2^22 for
 * float32), one copy per GPU, held until the process ends.  The call
 * allocates nothing; its first call on a device looks up that device's copy
 * (with the device current).  Arguments, layouts, outputs and errors as fa_bwd,
 * on the current device's stream `stream`, plus FA_ERR_SCRATCH when
 * fa_bwd_workspace_bytes(...) exceeds FA_NOALLOC_SCRATCH_BYTES (checked before
 * any device work) and FA_ERR_LAUNCH if the runtime cannot provide the
 * array's address.  Every call on one GPU uses the same array: calls that
 * overlap on one GPU (two streams, two host threads) race.  The array's
 * contents on entry do not matter (each call writes what it reads).
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* lse, void* dQ, void* dK, void* dV,
                   int B, int H, int Tq, int Tk, int d, float scale, int causal,
                   int dtype, int o_dtype, int grad_dtype, void* stream);

/*
 * Split-key forward for few query rows per head (decoding) -- the same
 * operation as fa_fwd, for bf16 inputs and d in {64, 128}.  With one or a few
 * queries per head the query-block grid is too small to fill the GPU, so the
 * keys of each head are also split into `nsplit` chunks; every chunk yields
 * partial results (running maximum, weight sums, unnormalised O) that a second
 * pass merges with the online-softmax rule ([Atlas] "Online softmax: the trick
 * that makes tiling exact"; [ZtF] "The forward pass", steps 2.3-2.5).
 *   nsplit     number of key chunks per 32-query block; 0 lets the library
 *              choose (a fixed function of B, H, Tq, Tk)
 *   workspace  device buffer of at least fa_fwd_splitkv_workspace_bytes(...)
 *              bytes for the partials, owned by the caller, contents on entry
 *              irrelevant
 * Other arguments, layouts and outputs as fa_fwd.  Errors as fa_fwd, plus
 * FA_ERR_DTYPE for float32 inputs, FA_ERR_HEADDIM for d = 256, FA_ERR_SHAPE for
 * nsplit < 0 and FA_ERR_WORKSPACE for a missing or short workspace.  The
 * partials are merged in a fixed order: results repeat bit for bit.
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Tq, int Tk, int d, int nsplit);
int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* lse,
                   int B, int H, int Tq, int Tk, int d, float scale, int causal,
                   int dtype, int out_dtype, int nsplit, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Block-sparse attention ([ZtF] "Dropout, block-sparsity, and other real-kernel
 * details"): the same operation as fa_fwd / fa_bwd restricted to the (query
 * block, key block) tiles a block mask keeps.  Every score outside a kept tile
 * is -inf, exactly as if it were masked out of the dense definition; causal
 * masking, when asked for, applies on top.  Tiles the mask drops are never
 * read or computed, so work and HBM traffic scale with the mask's density.
 *   block_mask  device buffer of uint8 [mask_heads][ceil(Tq/128)][ceil(Tk/128)],
 *               row-major; entry (h, i, j) != 0 keeps query rows 128i..128i+127
 *               against keys 128j..128j+127 for head h (for every batch entry).
 *               Owned by the caller, read only.
 *   mask_heads  1 (one mask shared by all heads) or H (one per head)
 * A query row whose mask row keeps no key (or, causal, no key at or before it)
 * gets O = 0 and lse = -inf, and its dQ is 0; keys no kept row sees get dK =
 * dV = 0.  bfloat16 inputs only.  Other
 * arguments, layouts, workspace and outputs as fa_fwd / fa_bwd.  Errors as
 * those, plus FA_ERR_NULL for a missing mask, FA_ERR_SHAPE for mask_heads not
 * in {1, H} and FA_ERR_DTYPE for float32 inputs.  Results repeat bit for bit.
 */
int fa_fwd_masked(const void* Q, const void* K, const void* V, void* O, float* lse,
                  int B, int H, int Tq, int Tk, int d, float scale, int causal,
                  int dtype, int out_dtype, const unsigned char* block_mask, int mask_heads,
                  void* stream);
int fa_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                  const float* lse, void* dQ, void* dK, void* dV,
                  int B, int H, int Tq, int Tk, int d, float scale, int causal,
                  int dtype, int o_dtype, int grad_dtype, const unsigned char* block_mask,
                  int mask_heads, void* workspace, size_t workspace_bytes, void* stream);
/* fa_bwd_masked split into phases, as fa_bwd_phases splits fa_bwd (same bits,
 * order, workspace contract and FA_ERR_PHASE). */
int fa_bwd_masked_phases(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* lse, void* dQ, void* dK, void* dV,
                         int B, int H, int Tq, int Tk, int d, float scale, int causal,
                         int dtype, int o_dtype, int grad_dtype, const unsigned char* block_mask,
                         int mask_heads, void* workspace, size_t workspace_bytes, int phases,
                         void* stream);

/*
 * Sliding-window attention ([ZtF] "Dropout, block-sparsity, and other
 * real-kernel details": windows are masks that are functions of (r, l)): the
 * same operation as fa_fwd / fa_bwd with key l visible from query r iff
 *   r - window_left <= l <= r + window_right,
 * each side >= 0, or -1 for unbounded (top-left alignment, as for causal).
 * (-1, 0) is causal attention and (-1, -1) full attention; they run the
 * corresponding fa_fwd / fa_bwd kernels.  Key blocks wholly outside a query
 * block's band (and query tiles outside a key block's) are never read or
 * computed, so work grows with the window, not with Tk.  A query row that
 * sees no key (possible when Tq > Tk + window_left) gets O = 0 and lse =
 * -inf, and its dQ is 0.  bfloat16 inputs only.  Other arguments, layouts,
 * workspace and outputs as fa_fwd / fa_bwd / fa_bwd_phases.  Errors as those,
 * plus FA_ERR_SHAPE for a side below -1 and FA_ERR_DTYPE for float32 inputs.
 * Results repeat bit for bit.
 */
int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* lse,
                  int B, int H, int Tq, int Tk, int d, float scale,
                  int window_left, int window_right, int dtype, int out_dtype, void* stream);
int fa_bwd_window(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                  const float* lse, void* dQ, void* dK, void* dV,
                  int B, int H, int Tq, int Tk, int d, float scale,
                  int window_left, int window_right, int dtype, int o_dtype, int grad_dtype,
                  void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_window_phases(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* lse, void* dQ, void* dK, void* dV,
                         int B, int H, int Tq, int Tk, int d, float scale,
                         int window_left, int window_right, int dtype, int o_dtype, int grad_dtype,
                         void* workspace, size_t workspace_bytes, int phases, void* stream);

/*
 * Document masks for packed sequences ([ZtF] "Dropout, block-sparsity, and
 * other real-kernel details": document masks are masks that are functions of
 * (r, l)): each of the B x H sequences of length T holds ndocs documents laid
 * end to end, and query r sees key l iff both lie in the same document (and,
 * when causal != 0, l <= r), i.e. attention runs on every document on its own.
 *   cu_seqlens  device buffer of int32 [ndocs + 1], 4-byte aligned: document i
 *               holds positions cu_seqlens[i] .. cu_seqlens[i+1] - 1, with
 *               cu_seqlens[0] = 0, non-decreasing, cu_seqlens[ndocs] = T
 *               (empty documents allowed).  One set of offsets serves every
 *               batch entry and head.  Owned by the caller, read only.
 *   ndocs       number of documents, >= 1
 * The library reads the offsets only on the device and cannot check them: with
 * offsets that break the rules above results are unspecified, but every memory
 * access stays inside the buffers.  Key blocks outside a query block's
 * documents (and query tiles outside a key block's) are never read or computed,
 * so work grows with the document lengths, not with T.  bfloat16 inputs only.
 * Other arguments (Tq = Tk = T), layouts, workspace and outputs as fa_fwd /
 * fa_bwd / fa_bwd_phases.  Errors as those, plus FA_ERR_NULL for a missing
 * cu_seqlens, FA_ERR_SHAPE for ndocs < 1, FA_ERR_ALIGN for a misaligned
 * cu_seqlens and FA_ERR_DTYPE for float32 inputs.  Results repeat bit for bit.
 */
int fa_fwd_docs(const void* Q, const void* K, const void* V, void* O, float* lse,
                int B, int H, int T, int d, float scale, int causal,
                const int* cu_seqlens, int ndocs, int dtype, int out_dtype, void* stream);
int fa_bwd_docs(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* lse, void* dQ, void* dK, void* dV,
                int B, int H, int T, int d, float scale, int causal,
                const int* cu_seqlens, int ndocs, int dtype, int o_dtype, int grad_dtype,
                void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_docs_phases(const void* Q, const void* K, const void* V, const void* O,
                       const void* dO, const float* lse, void* dQ, void* dK, void* dV,
                       int B, int H, int T, int d, float scale, int causal,
                       const int* cu_seqlens, int ndocs, int dtype, int o_dtype, int grad_dtype,
                       void* workspace, size_t workspace_bytes, int phases, void* stream);

/* Static, human-readable text for an fa_status value (never NULL). */
const char* fa_strerror(int status);

/* ABI version of this header (incremented on incompatible changes). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
