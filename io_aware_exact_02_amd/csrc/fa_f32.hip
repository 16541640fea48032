// float32 forward and backward (no downcast anywhere: float32 products and
// accumulation on the vector ALUs), plus the D pre-pass shared by both dtypes.
//
// [ZtF] = "FlashAttention", zerotofrontier.app textbook section 12.3.
//
// A group of G = D/16 lanes owns one row; lane j of a group holds features
// j, j+G, j+2G, ... so the group's LDS reads of a K/V row are G consecutive
// words (broadcast across groups, no bank conflicts).  Dot products are
// finished with xor-shuffles inside the group.
//
// Forward: FlashAttention-2 order ([ZtF] "The forward pass"), 32-key tiles in
// LDS, online softmax in log2 units.  Backward ([ZtF] "The backward pass,
// derived"): D = rowsum(dO * O) first, then one kernel with key rows outside
// (dK, dV accumulated in registers, written once) and one with query rows
// outside (dQ accumulated in registers, written once); both recompute
// P = exp(S - lse).  Splitting dQ into its own sweep avoids atomics, so the
// float32 gradients are deterministic.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kTileKeys = 32;
constexpr int kTileRows = 32;

template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// ------------------------------- forward -----------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, float* __restrict__ O,
                                                     float* __restrict__ lse, int Tq, int Tk, float cl2e,
                                                     int nqb) {
  constexpr int G = D / 16, E = 16, ROWS = 256 / G;
  __shared__ float Ks[kTileKeys][D];
  __shared__ float Vs[kTileKeys][D];
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int tid = threadIdx.x, j = tid % G, row = qb * ROWS + tid / G;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  float q[E], o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = row < Tq ? Q[qbase + (size_t)row * D + e * G + j] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  int last_key = Tk - 1;
  if (CAUSAL) last_key = min(last_key, min(qb * ROWS + ROWS, Tq) - 1);
  for (int k0 = 0; k0 <= last_key; k0 += kTileKeys) {
    __syncthreads();
    for (int x = tid; x < kTileKeys * D; x += 256) {
      const int kk = x / D, c = x % D, key = k0 + kk;
      Ks[kk][c] = key < Tk ? K[kbase + (size_t)key * D + c] : 0.f;
      Vs[kk][c] = key < Tk ? V[kbase + (size_t)key * D + c] : 0.f;
    }
    __syncthreads();
    float s[kTileKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kTileKeys; ++kk) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part = __builtin_fmaf(q[e], Ks[kk][e * G + j], part);
      float sv = group_sum<G>(part) * cl2e;
      const int key = k0 + kk;
      if (key >= Tk || (CAUSAL && key > row)) sv = -INFINITY;
      s[kk] = sv;
      mx = fmaxf(mx, sv);
    }
    const float m_new = fmaxf(m, mx);
    const float ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - ref);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kTileKeys; ++kk) {
      const float p = fast_exp2(s[kk] - ref);
      l += p;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(p, Vs[kk][e * G + j], o[e]);
    }
    m = m_new;
  }
  if (row >= Tq) return;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) O[qbase + (size_t)row * D + e * G + j] = o[e] * inv;
  if (j == 0) lse[(size_t)bh * Tq + row] = (m + log2f(l)) * kLn2;
}

// ------------------------------- D pre-pass --------------------------------
// D_r = dO_r . O_r in float32 ([ZtF] "The backward pass, derived", Observation 2).
template <int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const float* __restrict__ dO, const float* __restrict__ Ov,
                                                    float* __restrict__ Dout, long long rows) {
  constexpr int G = 16, E = D / G;
  const long long r = (long long)blockIdx.x * (256 / G) + threadIdx.x / G;
  const int j = threadIdx.x % G;
  float part = 0.f;
  if (r < rows) {
    const float* a = dO + r * D;
    const float* b = Ov + r * D;
#pragma unroll
    for (int e = 0; e < E; ++e) part = __builtin_fmaf(a[e * G + j], b[e * G + j], part);
  }
  part = group_sum<G>(part);
  if (r < rows && j == 0) Dout[r] = part;
}

// ----------------------- backward: key rows outside ------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_kv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V, const float* __restrict__ dO,
                                                        const float* __restrict__ lse, const float* __restrict__ Dr,
                                                        float* __restrict__ dK, float* __restrict__ dV, int Tq,
                                                        int Tk, float scale, int nkb) {
  constexpr int G = D / 16, E = 16, KEYS = 256 / G;
  __shared__ float Qs[kTileRows][D];
  __shared__ float dOs[kTileRows][D];
  __shared__ float Ls[kTileRows], Ds[kTileRows];
  const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int tid = threadIdx.x, j = tid % G, key = kb * KEYS + tid / G;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  float kr[E], vr[E], dk[E], dv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kr[e] = key < Tk ? K[kbase + (size_t)key * D + e * G + j] : 0.f;
    vr[e] = key < Tk ? V[kbase + (size_t)key * D + e * G + j] : 0.f;
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const int first_row = CAUSAL ? (kb * KEYS / kTileRows) * kTileRows : 0;
  for (int r0 = first_row; r0 < Tq; r0 += kTileRows) {
    __syncthreads();
    for (int x = tid; x < kTileRows * D; x += 256) {
      const int rr = x / D, c = x % D, row = r0 + rr;
      Qs[rr][c] = row < Tq ? Q[qbase + (size_t)row * D + c] : 0.f;
      dOs[rr][c] = row < Tq ? dO[qbase + (size_t)row * D + c] : 0.f;
    }
    if (tid < kTileRows) {
      const int row = r0 + tid;
      Ls[tid] = row < Tq ? lse[(size_t)bh * Tq + row] : 0.f;
      Ds[tid] = row < Tq ? Dr[(size_t)bh * Tq + row] : 0.f;
    }
    __syncthreads();
    for (int rr = 0; rr < kTileRows; ++rr) {
      const int row = r0 + rr;
      float ps = 0.f, pd = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ps = __builtin_fmaf(Qs[rr][e * G + j], kr[e], ps);
        pd = __builtin_fmaf(dOs[rr][e * G + j], vr[e], pd);
      }
      ps = group_sum<G>(ps);
      pd = group_sum<G>(pd);
      const bool vis = row < Tq && key < Tk && (!CAUSAL || key <= row);
      const float p = vis ? expf(scale * ps - Ls[rr]) : 0.f;
      const float ds = p * (pd - Ds[rr]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dv[e] = __builtin_fmaf(p, dOs[rr][e * G + j], dv[e]);
        dk[e] = __builtin_fmaf(ds, Qs[rr][e * G + j], dk[e]);
      }
    }
  }
  if (key >= Tk) return;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dK[kbase + (size_t)key * D + e * G + j] = scale * dk[e];
    dV[kbase + (size_t)key * D + e * G + j] = dv[e];
  }
}

// ----------------------- backward: query rows outside ----------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_q_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       const float* __restrict__ lse, const float* __restrict__ Dr,
                                                       float* __restrict__ dQ, int Tq, int Tk, float scale,
                                                       int nqb) {
  constexpr int G = D / 16, E = 16, ROWS = 256 / G;
  __shared__ float Ks[kTileKeys][D];
  __shared__ float Vs[kTileKeys][D];
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int tid = threadIdx.x, j = tid % G, row = qb * ROWS + tid / G;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  float q[E], g[E], dq[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = row < Tq ? Q[qbase + (size_t)row * D + e * G + j] : 0.f;
    g[e] = row < Tq ? dO[qbase + (size_t)row * D + e * G + j] : 0.f;
    dq[e] = 0.f;
  }
  const float L = row < Tq ? lse[(size_t)bh * Tq + row] : 0.f;
  const float Dv = row < Tq ? Dr[(size_t)bh * Tq + row] : 0.f;
  int last_key = Tk - 1;
  if (CAUSAL) last_key = min(last_key, min(qb * ROWS + ROWS, Tq) - 1);
  for (int k0 = 0; k0 <= last_key; k0 += kTileKeys) {
    __syncthreads();
    for (int x = tid; x < kTileKeys * D; x += 256) {
      const int kk = x / D, c = x % D, key = k0 + kk;
      Ks[kk][c] = key < Tk ? K[kbase + (size_t)key * D + c] : 0.f;
      Vs[kk][c] = key < Tk ? V[kbase + (size_t)key * D + c] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < kTileKeys; ++kk) {
      const int key = k0 + kk;
      float ps = 0.f, pd = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ps = __builtin_fmaf(q[e], Ks[kk][e * G + j], ps);
        pd = __builtin_fmaf(g[e], Vs[kk][e * G + j], pd);
      }
      ps = group_sum<G>(ps);
      pd = group_sum<G>(pd);
      const bool vis = row < Tq && key < Tk && (!CAUSAL || key <= row);
      const float p = vis ? expf(scale * ps - L) : 0.f;
      const float ds = p * (pd - Dv);
#pragma unroll
      for (int e = 0; e < E; ++e) dq[e] = __builtin_fmaf(ds, Ks[kk][e * G + j], dq[e]);
    }
  }
  if (row >= Tq) return;
#pragma unroll
  for (int e = 0; e < E; ++e) dQ[qbase + (size_t)row * D + e * G + j] = scale * dq[e];
}

template <int D>
int fwd_f32(const float* Q, const float* K, const float* V, float* O, float* lse, int B, int H, int Tq, int Tk,
            float scale, int causal, hipStream_t stream) {
  constexpr int ROWS = 256 / (D / 16);
  const int nqb = (Tq + ROWS - 1) / ROWS;
  const long long nblk = (long long)nqb * B * H;
  if (nblk > 0x7fffffffLL) return FA_ERR_SHAPE;
  const float cl2e = scale * kLog2e;
  if (causal)
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3((unsigned)nblk), dim3(256), 0, stream, Q, K, V, O, lse, Tq, Tk,
                       cl2e, nqb);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3((unsigned)nblk), dim3(256), 0, stream, Q, K, V, O, lse, Tq,
                       Tk, cl2e, nqb);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int D>
int bwd_f32(const float* Q, const float* K, const float* V, const float* Ov, const float* dO, const float* lse,
            float* dQ, float* dK, float* dV, int B, int H, int Tq, int Tk, float scale, int causal, float* Dws,
            int phases, hipStream_t stream) {
  constexpr int ROWS = 256 / (D / 16);
  const long long rows = (long long)B * H * Tq;
  const long long nrd = (rows + 15) / 16;
  const int nqb = (Tq + ROWS - 1) / ROWS, nkb = (Tk + ROWS - 1) / ROWS;
  const long long nq = (long long)nqb * B * H, nk = (long long)nkb * B * H;
  if (nrd > 0x7fffffffLL || nq > 0x7fffffffLL || nk > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (phases & FA_BWD_PRE)
    hipLaunchKernelGGL((rowdot_kernel<D>), dim3((unsigned)nrd), dim3(256), 0, stream, dO, Ov, Dws, rows);
  if (phases & FA_BWD_MAIN) {   // key-block sweep: dK, dV
    if (causal)
      hipLaunchKernelGGL((bwd_kv_f32_kernel<D, true>), dim3((unsigned)nk), dim3(256), 0, stream, Q, K, V, dO, lse,
                         Dws, dK, dV, Tq, Tk, scale, nkb);
    else
      hipLaunchKernelGGL((bwd_kv_f32_kernel<D, false>), dim3((unsigned)nk), dim3(256), 0, stream, Q, K, V, dO, lse,
                         Dws, dK, dV, Tq, Tk, scale, nkb);
  }
  if (phases & FA_BWD_POST) {   // query-block sweep: dQ
    if (causal)
      hipLaunchKernelGGL((bwd_q_f32_kernel<D, true>), dim3((unsigned)nq), dim3(256), 0, stream, Q, K, V, dO, lse,
                         Dws, dQ, Tq, Tk, scale, nqb);
    else
      hipLaunchKernelGGL((bwd_q_f32_kernel<D, false>), dim3((unsigned)nq), dim3(256), 0, stream, Q, K, V, dO, lse,
                         Dws, dQ, Tq, Tk, scale, nqb);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int launch_fwd_f32(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq,
                   int Tk, int d, float scale, int causal, hipStream_t stream) {
  auto q = static_cast<const float*>(Q);
  auto k = static_cast<const float*>(K);
  auto v = static_cast<const float*>(V);
  auto o = static_cast<float*>(O);
  switch (d) {
    case 64: return fwd_f32<64>(q, k, v, o, lse, B, H, Tq, Tk, scale, causal, stream);
    case 128: return fwd_f32<128>(q, k, v, o, lse, B, H, Tq, Tk, scale, causal, stream);
    case 256: return fwd_f32<256>(q, k, v, o, lse, B, H, Tq, Tk, scale, causal, stream);
    default: return FA_ERR_HEADDIM;
  }
}

int launch_bwd_f32(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                   void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal,
                   void* workspace, int phases, hipStream_t stream) {
  auto q = static_cast<const float*>(Q);
  auto k = static_cast<const float*>(K);
  auto v = static_cast<const float*>(V);
  auto o = static_cast<const float*>(O);
  auto g = static_cast<const float*>(dO);
  auto dq = static_cast<float*>(dQ);
  auto dk = static_cast<float*>(dK);
  auto dv = static_cast<float*>(dV);
  auto ws = static_cast<float*>(workspace);
  switch (d) {
    case 64: return bwd_f32<64>(q, k, v, o, g, lse, dq, dk, dv, B, H, Tq, Tk, scale, causal, ws, phases, stream);
    case 128: return bwd_f32<128>(q, k, v, o, g, lse, dq, dk, dv, B, H, Tq, Tk, scale, causal, ws, phases, stream);
    case 256: return bwd_f32<256>(q, k, v, o, g, lse, dq, dk, dv, B, H, Tq, Tk, scale, causal, ws, phases, stream);
    default: return FA_ERR_HEADDIM;
  }
}

}  // namespace fa
