// C-ABI entry points of libfa.so: argument checks, dispatch on (dtype, d), launches.
// Every check runs before any device work; nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include "fa.h"
#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_d(int d) { return d == 64 || d == 128 || d == 256; }
bool valid_dtype(int t) { return t == FA_F32 || t == FA_BF16; }

int check_common(int B, int H, int Tq, int Tk, int d, float scale, int dtype) {
  if (B < 1 || H < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
  if (!valid_d(d)) return FA_ERR_HEADDIM;
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  // element offsets are 64-bit inside the kernels; guard the products anyway
  // one (batch, head) slice must stay below 2 GiB: the kernels address a slice
  // with 32-bit byte offsets (buffer resources)
  const long long bh = (long long)B * H;
  const long long tmax = Tq > Tk ? Tq : Tk;
  if (bh > (1LL << 31) || tmax * d * 4 >= (1LL << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

// block mask [mask_heads][ceil(Tq/128)][ceil(Tk/128)] bytes
int check_mask(const unsigned char* block_mask, int mask_heads, int H, int dtype) {
  if (!block_mask) return FA_ERR_NULL;
  if (mask_heads != 1 && mask_heads != H) return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  return FA_OK;
}

// sliding window (wl, wr): each side >= 0, or -1 for unbounded
int check_window(int wl, int wr, int dtype) {
  if (wl < -1 || wr < -1) return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  return FA_OK;
}

// An unbounded window side becomes a bound past any index (sequences are below 2^24).
int window_side(int w) { return w < 0 ? (1 << 30) : w; }

// The window kernels serve proper windows; (-1, -1) is full attention and (-1, 0)
// causal, which the dense kernels handle.  Returns 1 if the window kernels apply,
// and sets causal for the other two.
int window_mode(int wl, int wr, int* causal) {
  *causal = (wl < 0 && wr == 0) ? 1 : 0;
  return !(wl < 0 && (wr < 0 || wr == 0));
}

// documents of a packed sequence: offsets cu_seqlens[0 .. ndocs] on the device
int check_docs(const int* cu_seqlens, int ndocs, int dtype) {
  if (!cu_seqlens) return FA_ERR_NULL;
  if (ndocs < 1) return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return FA_ERR_ALIGN;
  return FA_OK;
}

int bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse, void* dQ,
             void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal, int dtype,
             int o_dtype, int grad_dtype, const unsigned char* block_mask, int mask_heads, void* workspace,
             size_t workspace_bytes, int phases, void* stream, int band = 0, int wl = 0, int wr = 0,
             const int* cu = nullptr, int nd = 0);

}  // namespace

namespace fa {

// The checks of fa_bwd that do not involve the workspace, in the same order.
int check_bwd_args(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                   void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int dtype,
                   int o_dtype, int grad_dtype) {
  if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV) return FA_ERR_NULL;
  int st = check_common(B, H, Tq, Tk, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!valid_dtype(grad_dtype) || (dtype == FA_F32 && grad_dtype != FA_F32)) return FA_ERR_DTYPE;
  if (!valid_dtype(o_dtype) || (dtype == FA_F32 && o_dtype != FA_F32)) return FA_ERR_DTYPE;
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  return FA_OK;
}

}  // namespace fa

extern "C" {

int fa_abi_version(void) { return 1; }

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: B, H, Tq and Tk must be >= 1 and the grid must fit";
    case FA_ERR_HEADDIM: return "unsupported head dimension (supported: 64, 128, 256)";
    case FA_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than the *_workspace_bytes() size";
    case FA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case FA_ERR_ALIGN: return "device pointers must be 16-byte aligned";
    case FA_ERR_PHASE: return "unknown bits in the backward phase mask";
    case FA_ERR_SCRATCH: return "problem too large for the library's static scratch (fa_bwd_noalloc)";
    default: return "unknown fa_status";
  }
}

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq, int Tk,
           int d, float scale, int causal, int dtype, int out_dtype, void* stream) {
  if (!Q || !K || !V || !O || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, Tq, Tk, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!valid_dtype(out_dtype) || (dtype == FA_F32 && out_dtype != FA_F32)) return FA_ERR_DTYPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(lse)) return FA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  causal = causal ? 1 : 0;
  if (dtype == FA_BF16)
    return fa::launch_fwd_bf16(Q, K, V, O, lse, B, H, Tq, Tk, d, scale, causal, out_dtype == FA_F32 ? 1 : 0, s);
  return fa::launch_fwd_f32(Q, K, V, O, lse, B, H, Tq, Tk, d, scale, causal, s);
}

size_t fa_bwd_workspace_bytes(int B, int H, int Tq, int Tk, int d, int dtype, int grad_dtype) {
  if (check_common(B, H, Tq, Tk, d, 1.f, dtype) != FA_OK || !valid_dtype(grad_dtype)) return 0;
  const long long rows = (long long)B * H * Tq;
  long long floats = fa::bwd_rows_padded(rows);                 // D (fp32 inputs) or -D (bf16)
  if (dtype == FA_BF16) floats += fa::bwd_rows_padded(rows);      // -lse log2 e
  return (size_t)floats * sizeof(float);
}

int fa_bwd_phases(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                  void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal,
                  int dtype, int o_dtype, int grad_dtype, void* workspace, size_t workspace_bytes, int phases,
                  void* stream) {
  return bwd_impl(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, causal, dtype, o_dtype, grad_dtype,
                  nullptr, 1, workspace, workspace_bytes, phases, stream);
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse, void* dQ,
           void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal, int dtype,
           int o_dtype, int grad_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_phases(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, causal, dtype, o_dtype,
                       grad_dtype, workspace, workspace_bytes, FA_BWD_ALL, stream);
}

int fa_fwd_masked(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq, int Tk,
                  int d, float scale, int causal, int dtype, int out_dtype, const unsigned char* block_mask,
                  int mask_heads, void* stream) {
  if (!Q || !K || !V || !O || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, Tq, Tk, d, scale, dtype);
  if (st != FA_OK) return st;
  st = check_mask(block_mask, mask_heads, H, dtype);
  if (st != FA_OK) return st;
  if (!valid_dtype(out_dtype)) return FA_ERR_DTYPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(lse)) return FA_ERR_ALIGN;
  return fa::launch_fwd_bf16(Q, K, V, O, lse, B, H, Tq, Tk, d, scale, causal ? 1 : 0, out_dtype == FA_F32 ? 1 : 0,
                             static_cast<hipStream_t>(stream), block_mask, mask_heads);
}

int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq, int Tk,
                  int d, float scale, int window_left, int window_right, int dtype, int out_dtype, void* stream) {
  if (!Q || !K || !V || !O || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, Tq, Tk, d, scale, dtype);
  if (st != FA_OK) return st;
  st = check_window(window_left, window_right, dtype);
  if (st != FA_OK) return st;
  if (!valid_dtype(out_dtype)) return FA_ERR_DTYPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(lse)) return FA_ERR_ALIGN;
  int causal = 0;
  const int win = window_mode(window_left, window_right, &causal);
  return fa::launch_fwd_bf16(Q, K, V, O, lse, B, H, Tq, Tk, d, scale, causal, out_dtype == FA_F32 ? 1 : 0,
                             static_cast<hipStream_t>(stream), nullptr, 1, win, window_side(window_left),
                             window_side(window_right));
}

int fa_bwd_window_phases(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                         const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d,
                         float scale, int window_left, int window_right, int dtype, int o_dtype, int grad_dtype,
                         void* workspace, size_t workspace_bytes, int phases, void* stream) {
  const int st = check_window(window_left, window_right, dtype);
  if (st != FA_OK) return st;
  int causal = 0;
  const int win = window_mode(window_left, window_right, &causal);
  return bwd_impl(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, causal, dtype, o_dtype, grad_dtype,
                  nullptr, 1, workspace, workspace_bytes, phases, stream, win, window_side(window_left),
                  window_side(window_right));
}

int fa_bwd_window(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                  void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int window_left,
                  int window_right, int dtype, int o_dtype, int grad_dtype, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return fa_bwd_window_phases(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, window_left, window_right,
                              dtype, o_dtype, grad_dtype, workspace, workspace_bytes, FA_BWD_ALL, stream);
}

int fa_fwd_docs(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int T, int d,
                float scale, int causal, const int* cu_seqlens, int ndocs, int dtype, int out_dtype, void* stream) {
  if (!Q || !K || !V || !O || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, T, T, d, scale, dtype);
  if (st != FA_OK) return st;
  st = check_docs(cu_seqlens, ndocs, dtype);
  if (st != FA_OK) return st;
  if (!valid_dtype(out_dtype)) return FA_ERR_DTYPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(lse)) return FA_ERR_ALIGN;
  return fa::launch_fwd_bf16(Q, K, V, O, lse, B, H, T, T, d, scale, causal ? 1 : 0, out_dtype == FA_F32 ? 1 : 0,
                             static_cast<hipStream_t>(stream), nullptr, 1, 2, 0, 0, cu_seqlens, ndocs);
}

int fa_bwd_docs_phases(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                       void* dQ, void* dK, void* dV, int B, int H, int T, int d, float scale, int causal,
                       const int* cu_seqlens, int ndocs, int dtype, int o_dtype, int grad_dtype, void* workspace,
                       size_t workspace_bytes, int phases, void* stream) {
  const int st = check_docs(cu_seqlens, ndocs, dtype);
  if (st != FA_OK) return st;
  return bwd_impl(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, T, T, d, scale, causal, dtype, o_dtype, grad_dtype,
                  nullptr, 1, workspace, workspace_bytes, phases, stream, 2, 0, 0, cu_seqlens, ndocs);
}

int fa_bwd_docs(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                void* dQ, void* dK, void* dV, int B, int H, int T, int d, float scale, int causal,
                const int* cu_seqlens, int ndocs, int dtype, int o_dtype, int grad_dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  return fa_bwd_docs_phases(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, T, d, scale, causal, cu_seqlens, ndocs, dtype,
                            o_dtype, grad_dtype, workspace, workspace_bytes, FA_BWD_ALL, stream);
}

int fa_bwd_masked_phases(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                         const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d,
                         float scale, int causal, int dtype, int o_dtype, int grad_dtype,
                         const unsigned char* block_mask, int mask_heads, void* workspace, size_t workspace_bytes,
                         int phases, void* stream) {
  if (!block_mask) return FA_ERR_NULL;
  return bwd_impl(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, causal, dtype, o_dtype, grad_dtype,
                  block_mask, mask_heads, workspace, workspace_bytes, phases, stream);
}

int fa_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                  void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal,
                  int dtype, int o_dtype, int grad_dtype, const unsigned char* block_mask, int mask_heads,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_masked_phases(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, causal, dtype, o_dtype,
                              grad_dtype, block_mask, mask_heads, workspace, workspace_bytes, FA_BWD_ALL, stream);
}

}  // extern "C"

namespace {

int bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse, void* dQ,
             void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal, int dtype,
             int o_dtype, int grad_dtype, const unsigned char* block_mask, int mask_heads, void* workspace,
             size_t workspace_bytes, int phases, void* stream, int band, int wl, int wr, const int* cu, int nd) {
  if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV) return FA_ERR_NULL;
  int st = check_common(B, H, Tq, Tk, d, scale, dtype);
  if (st != FA_OK) return st;
  if (block_mask) {
    st = check_mask(block_mask, mask_heads, H, dtype);
    if (st != FA_OK) return st;
  }
  if (!valid_dtype(grad_dtype) || (dtype == FA_F32 && grad_dtype != FA_F32)) return FA_ERR_DTYPE;
  if (!valid_dtype(o_dtype) || (dtype == FA_F32 && o_dtype != FA_F32)) return FA_ERR_DTYPE;
  if (phases & ~FA_BWD_ALL) return FA_ERR_PHASE;
  const size_t need = fa_bwd_workspace_bytes(B, H, Tq, Tk, d, dtype, grad_dtype);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if (phases == 0) return FA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  causal = causal ? 1 : 0;
  if (dtype == FA_BF16)
    return fa::launch_bwd_bf16(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, causal,
                               o_dtype == FA_F32 ? 1 : 0, grad_dtype == FA_F32 ? 1 : 0, workspace, phases, s,
                               block_mask, mask_heads, band, wl, wr, cu, nd);
  return fa::launch_bwd_f32(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, causal, workspace, phases, s);
}

}  // namespace

extern "C" {

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Tq, int Tk, int d, int nsplit) {
  if (check_common(B, H, Tq, Tk, d, 1.f, FA_BF16) != FA_OK || d == 256 || nsplit < 0) return 0;
  const long long parts = 4LL * fa::splitkv_parts(B, H, Tq, Tk, nsplit);
  const long long rows = (long long)B * H * Tq;
  return (size_t)(parts * rows * (d + 4) * (long long)sizeof(float));
}

int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq, int Tk,
                   int d, float scale, int causal, int dtype, int out_dtype, int nsplit, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!Q || !K || !V || !O || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, Tq, Tk, d, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16 || !valid_dtype(out_dtype)) return FA_ERR_DTYPE;
  if (d == 256) return FA_ERR_HEADDIM;
  if (nsplit < 0) return FA_ERR_SHAPE;
  const size_t need = fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, d, nsplit);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {Q, K, V, O, lse, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  return fa::launch_decode_bf16(Q, K, V, O, lse, B, H, Tq, Tk, d, scale, causal ? 1 : 0,
                                out_dtype == FA_F32 ? 1 : 0, fa::splitkv_parts(B, H, Tq, Tk, nsplit), workspace,
                                static_cast<hipStream_t>(stream));
}

}  // extern "C"
