// Internal launchers shared by the C-ABI entry points (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include "fa.h"

namespace fa {

// Workspace layout of fa_bwd: float32 row terms D [rows] padded to a multiple of
// 64 floats (256 bytes), then (bf16 gradients only) the float32 dQ accumulator.
inline long long bwd_rows_padded(long long rows) { return (rows + 63) / 64 * 64; }

// fa_bwd's argument checks that do not involve the workspace (null pointers,
// shape, head width, dtypes, scale, 16-byte alignment), in fa_bwd's order.
int check_bwd_args(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                   void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int dtype,
                   int o_dtype, int grad_dtype);

// bmask: optional block mask [mask_heads][ceil(Tq/128)][ceil(Tk/128)] (uint8, device memory)
// band 1: sliding window, key l visible from query r iff r - wl <= l <= r + wr
// (wl, wr >= 0; an unbounded side is passed as a large value).  band 2:
// documents of a packed sequence, offsets cu[0..nd] on the device, causal
// within each document when causal != 0.
int launch_fwd_bf16(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq,
                    int Tk, int d, float scale, int causal, int out_f32, hipStream_t stream,
                    const uint8_t* bmask = nullptr, int mask_heads = 1, int band = 0, int wl = 0, int wr = 0,
                    const int* cu = nullptr, int nd = 0);
int launch_fwd_f32(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq,
                   int Tk, int d, float scale, int causal, hipStream_t stream);
int launch_bwd_bf16(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                    void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal,
                    int o_f32, int grad_f32, void* workspace, int phases, hipStream_t stream,
                    const uint8_t* bmask = nullptr, int mask_heads = 1, int band = 0, int wl = 0, int wr = 0,
                    const int* cu = nullptr, int nd = 0);
int launch_bwd_f32(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                   void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal,
                   void* workspace, int phases, hipStream_t stream);
// Split-key forward for few query rows: nsplit key chunks per 32-query block,
// four partials per chunk (one per wave); splitkv_parts resolves nsplit = 0.
int splitkv_parts(int B, int H, int Tq, int Tk, int nsplit);
int launch_decode_bf16(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq,
                       int Tk, int d, float scale, int causal, int out_f32, int nsplit, void* workspace,
                       hipStream_t stream);

}  // namespace fa
