// Backward pass for bf16 inputs on gfx950 MFMA.
//
// [ZtF] = "FlashAttention", zerotofrontier.app textbook section 12.3,
// sections "The backward pass, derived" and "Which loop goes outside?".
//
// One workgroup owns a block of 128 keys of one (batch, head); each of its
// four waves owns 32 of them and keeps K_j, V_j (as MFMA B operands) and the
// float32 accumulators dK_j, dV_j in registers for the whole sweep over query
// blocks of 32 rows (causal: starting at the first query that can see the
// block).  Per query block i:
//   * Q_i and dO_i are read from HBM once (16-byte loads, prefetched into
//     registers one block ahead) and written to LDS twice: row-major for the
//     products that contract over the feature axis, and transposed (query
//     order permuted to match the MFMA k-slots) for the ones that contract
//     over queries.  lse_i and D_i go to LDS as well.
//   * S = Q_i K_j^T on MFMA with one key per lane (Observation 1: the weights
//     are rebuilt as P = exp2(S * scale*log2e - lse*log2e), masked on the
//     causal diagonal and the tails).
//   * dV_j += P^T dO_i; dP = dO_i V_j^T; dS = P * (dP - D_i) (Observation 3);
//     dK_j += dS^T Q_i -- all on MFMA with P and dS taken from registers.
//   * dS (bf16) goes to LDS; the workgroup then forms dQ_i's contribution of
//     all 128 keys, scale * dS K_j, and adds it to a float32 accumulator in
//     HBM with atomic adds (the order of additions from different key blocks
//     is not fixed, so dQ's last bits may vary between runs).
// Before the sweep, a pre-pass writes D = rowsum(dO * O) (Observation 2) and
// clears the dQ accumulator; afterwards, if the caller wants bf16 dQ, a
// post-pass rounds the accumulator.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kKeysPerWave = 32;
constexpr int kWavesB = 4;
constexpr int kBKC = kKeysPerWave * kWavesB;   // keys per workgroup
constexpr int kBQ = 32;                        // query rows per step

template <int D>
struct BwdLayout {
  static constexpr int NSTR = D + 8;        // row-major tiles (bf16 per row)
  static constexpr int TSTR = kBQ + 8;      // transposed Q/dO tiles: D rows of 32 queries
  static constexpr int KTSTR = kBKC + 8;    // transposed K tile: D rows of 128 keys
  static constexpr int SSTR = kBKC + 8;     // dS tile: 32 rows of 128 keys
  static constexpr int QN = kBQ * NSTR;     // Q row-major
  static constexpr int QT = D * TSTR;       // Q transposed
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_QT = OFF_Q + QN;
  static constexpr int OFF_G = OFF_QT + QT;     // dO row-major
  static constexpr int OFF_GT = OFF_G + QN;     // dO transposed
  static constexpr int OFF_KT = OFF_GT + QT;    // K transposed (whole key block)
  static constexpr int OFF_S = OFF_KT + D * KTSTR;
  static constexpr int OFF_F = OFF_S + kBQ * SSTR;   // float area: lse*log2e[32], D[32]
  static constexpr int ELEMS = OFF_F + 2 * kBQ * 2;  // in bf16 units
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NBLK = (kBQ / 8) * (D / 8);   // 8x8 blocks per tensor tile
  static_assert(OFF_F % 8 == 0, "float area must be 16-byte aligned");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float* __restrict__ lse, const float* __restrict__ Dr,
                     float* __restrict__ dQacc, void* __restrict__ dK, void* __restrict__ dV,
                     int Tq, int Tk, float scale, float cl2e, int nkb, int grad_f32) {
  using L = BwdLayout<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[L::ELEMS];
  uint16_t* Qs = smem + L::OFF_Q;
  uint16_t* QTs = smem + L::OFF_QT;
  uint16_t* Gs = smem + L::OFF_G;
  uint16_t* GTs = smem + L::OFF_GT;
  uint16_t* KTs = smem + L::OFF_KT;
  uint16_t* Ss = smem + L::OFF_S;
  float* Ls = reinterpret_cast<float*>(smem + L::OFF_F);
  float* Ds = Ls + kBQ;

  const int nblk = gridDim.x, wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int bh = lin / nkb;
  const int kblk = CAUSAL ? nkb - 1 - (lin % nkb) : (lin % nkb);   // causal: longest sweeps first
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hf = lane >> 5;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  const int k0 = kblk * kBKC;
  const int mykey = k0 + wave * kKeysPerWave + l32;

  // K_j and V_j as B operands (column = key, k = features), held for the sweep.
  bf16x8 kf[L::NDS], vf[L::NDS];
#pragma unroll
  for (int ds = 0; ds < L::NDS; ++ds) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (mykey < Tk) {
      a = ld16(K + kbase + (size_t)mykey * D + ds * 16 + 8 * hf);
      b = ld16(V + kbase + (size_t)mykey * D + ds * 16 + 8 * hf);
    }
    kf[ds] = as_bf16x8(a);
    vf[ds] = as_bf16x8(b);
  }
  // K_j^T for the dQ product: 8x8 blocks (8 keys x 8 features) transposed into LDS
  for (int b = tid; b < (kBKC / 8) * (D / 8); b += 256) {
    const int kg = b % (kBKC / 8), dg = b / (kBKC / 8);
    u32x4 r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = k0 + kg * 8 + i;
      r[i] = key < Tk ? ld16(K + kbase + (size_t)key * D + dg * 8) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x4 even, odd;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        even[p] = lo_lo(r[2 * p][w], r[2 * p + 1][w]);
        odd[p] = hi_hi(r[2 * p][w], r[2 * p + 1][w]);
      }
      st16(KTs + (dg * 8 + 2 * w) * L::KTSTR + kg * 8, even);
      st16(KTs + (dg * 8 + 2 * w + 1) * L::KTSTR + kg * 8, odd);
    }
  }

  f32x16 dk[L::NDB], dv[L::NDB];
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  const int nqt = (Tq + kBQ - 1) / kBQ;
  const int it0 = CAUSAL ? min(k0 / kBQ, nqt) : 0;

  // ---- staging of one query tile (Q_i, dO_i, lse_i, D_i) ----
  // threads [0, 2*NBLK): one 8x8 block of Q (first half) or dO (second half)
  const bool tloader = tid < 2 * L::NBLK;
  const int tb = tid % L::NBLK;
  const bool is_g = tid >= L::NBLK;
  const int rg = tb % (kBQ / 8), dgq = tb / (kBQ / 8);
  const int rt = rg >> 1, rh = rg & 1;
  auto trow = [&](int i) { return 16 * rt + 4 * rh + (i < 4 ? i : 4 + i); };
  u32x4 stg[8];
  float sl = 0.f, sd = 0.f;
  auto gload = [&](int it) {
    const int r0 = it * kBQ;
    if (tloader) {
      const uint16_t* src = is_g ? dO : Q;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = r0 + trow(i);
        stg[i] = row < Tq ? ld16(src + qbase + (size_t)row * D + dgq * 8) : (u32x4){0u, 0u, 0u, 0u};
      }
    }
    if (tid >= 256 - kBQ) {
      const int row = r0 + tid - (256 - kBQ);
      sl = row < Tq ? lse[(size_t)bh * Tq + row] * kLog2e : 0.f;
      sd = row < Tq ? Dr[(size_t)bh * Tq + row] : 0.f;
    }
  };
  auto lstore = [&]() {
    if (tloader) {
      uint16_t* N = is_g ? Gs : Qs;
      uint16_t* T = is_g ? GTs : QTs;
#pragma unroll
      for (int i = 0; i < 8; ++i) st16(N + trow(i) * L::NSTR + dgq * 8, stg[i]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 even, odd;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          even[p] = lo_lo(stg[2 * p][w], stg[2 * p + 1][w]);
          odd[p] = hi_hi(stg[2 * p][w], stg[2 * p + 1][w]);
        }
        st16(T + (dgq * 8 + 2 * w) * L::TSTR + 16 * rt + 8 * rh, even);
        st16(T + (dgq * 8 + 2 * w + 1) * L::TSTR + 16 * rt + 8 * rh, odd);
      }
    }
    if (tid >= 256 - kBQ) {
      Ls[tid - (256 - kBQ)] = sl;
      Ds[tid - (256 - kBQ)] = sd;
    }
  };

  if (it0 < nqt) {
    gload(it0);
    lstore();
  }
  __syncthreads();

  for (int it = it0; it < nqt; ++it) {
    const int r0 = it * kBQ;
    if (it + 1 < nqt) gload(it + 1);

    // S = Q_i K_j^T and dP = dO_i V_j^T: lane = key, register r = query 8(r/4)+4hf+r%4
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int ds = 0; ds < L::NDS; ++ds) {
      const bf16x8 a = as_bf16x8(ld16(Qs + l32 * L::NSTR + ds * 16 + 8 * hf));
      s = mfma32(a, kf[ds], s);
      const bf16x8 g = as_bf16x8(ld16(Gs + l32 * L::NSTR + ds * 16 + 8 * hf));
      dp = mfma32(g, vf[ds], dp);
    }
    float p[16], dsv[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int qr = 8 * g4 + 4 * hf;
      const f32x4 lv = *reinterpret_cast<const f32x4*>(Ls + qr);
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(Ds + qr);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g4 + e;
        const int q = r0 + qr + e;
        const bool vis = q < Tq && mykey < Tk && (!CAUSAL || mykey <= q);
        const float pv = vis ? fast_exp2(__builtin_fmaf(s[r], cl2e, -lv[e])) : 0.f;
        p[r] = pv;
        dsv[r] = pv * (dp[r] - dv4[e]);
      }
    }
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = pack_bf16(p[8 * t + 2 * e], p[8 * t + 2 * e + 1]);
        b[e] = pack_bf16(dsv[8 * t + 2 * e], dsv[8 * t + 2 * e + 1]);
      }
      pb[t] = as_bf16x8(a);
      sb[t] = as_bf16x8(b);
    }
    // dV_j += P^T dO_i ; dK_j += dS^T Q_i  (lane = feature column, register = key row)
#pragma unroll
    for (int db = 0; db < L::NDB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 g = as_bf16x8(ld16(GTs + (db * 32 + l32) * L::TSTR + 16 * t + 8 * hf));
        dv[db] = mfma32(pb[t], g, dv[db]);
        const bf16x8 qq = as_bf16x8(ld16(QTs + (db * 32 + l32) * L::TSTR + 16 * t + 8 * hf));
        dk[db] = mfma32(sb[t], qq, dk[db]);
      }
    // dS -> LDS as [query][key] (bf16) for the dQ product
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = 8 * (r >> 2) + 4 * hf + (r & 3);
      const unsigned w = pack_bf16(dsv[r], 0.f);
      Ss[qr * L::SSTR + wave * kKeysPerWave + l32] = (uint16_t)(w & 0xffffu);
    }
    __syncthreads();
    // dQ_i += scale * dS K_j over the workgroup's 128 keys; wave -> 32-feature blocks
    for (int db = wave; db < L::NDB; db += kWavesB) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kBKC / 16; ++ks) {
        const bf16x8 a = as_bf16x8(ld16(Ss + l32 * L::SSTR + ks * 16 + 8 * hf));
        const bf16x8 b = as_bf16x8(ld16(KTs + (db * 32 + l32) * L::KTSTR + ks * 16 + 8 * hf));
        acc = mfma32(a, b, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = r0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (q < Tq) atomicAdd(dQacc + qbase + (size_t)q * D + db * 32 + l32, scale * acc[r]);
      }
    }
    __syncthreads();
    if (it + 1 < nqt) lstore();
    __syncthreads();
  }

  // dK_j = scale * dS^T Q, dV_j: lane = feature, register r = key 8(r/4)+4hf+r%4
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + wave * kKeysPerWave + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key >= Tk) continue;
      const size_t off = kbase + (size_t)key * D + db * 32 + l32;
      const float gk = scale * dk[db][r], gv = dv[db][r];
      if (grad_f32) {
        static_cast<float*>(dK)[off] = gk;
        static_cast<float*>(dV)[off] = gv;
      } else {
        static_cast<uint16_t*>(dK)[off] = (uint16_t)(pack_bf16(gk, 0.f) & 0xffffu);
        static_cast<uint16_t*>(dV)[off] = (uint16_t)(pack_bf16(gv, 0.f) & 0xffffu);
      }
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, long long n) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    *reinterpret_cast<f32x4*>(p + i) = (f32x4){0.f, 0.f, 0.f, 0.f};
  } else {
    for (long long k = i; k < n; ++k) p[k] = 0.f;
  }
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                         long long n) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
    u32x2 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    st8(dst + i, w);
  } else {
    for (long long k = i; k < n; ++k) dst[k] = (uint16_t)(pack_bf16(src[k], 0.f) & 0xffffu);
  }
}

template <int D>
int bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse, void* dQ,
        void* dK, void* dV, int B, int H, int Tq, int Tk, float scale, int causal, int o_f32, int grad_f32,
        void* workspace, int phases, hipStream_t stream) {
  const long long rows = (long long)B * H * Tq;
  const long long nq = rows * D;
  const int nkb = (Tk + kBKC - 1) / kBKC;
  const long long nblk = (long long)nkb * B * H;
  const long long nfill = (nq + 1023) / 1024;
  if (nblk > 0x7fffffffLL || nfill > 0x7fffffffLL) return FA_ERR_SHAPE;
  float* Dws = static_cast<float*>(workspace);
  float* acc = grad_f32 ? static_cast<float*>(dQ) : Dws + bwd_rows_padded(rows);
  if (phases & FA_BWD_PRE) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)nfill), dim3(256), 0, stream, acc, nq);
    const int st = launch_rowdot_bf16(dO, O, o_f32, Dws, rows, D, stream);
    if (st != FA_OK) return st;
  }
  if (phases & FA_BWD_MAIN) {
    const float cl2e = scale * kLog2e;
    auto q = static_cast<const uint16_t*>(Q);
    auto k = static_cast<const uint16_t*>(K);
    auto v = static_cast<const uint16_t*>(V);
    auto g = static_cast<const uint16_t*>(dO);
    if (causal)
      hipLaunchKernelGGL((bwd_bf16_kernel<D, true>), dim3((unsigned)nblk), dim3(256), 0, stream, q, k, v, g, lse,
                         Dws, acc, dK, dV, Tq, Tk, scale, cl2e, nkb, grad_f32);
    else
      hipLaunchKernelGGL((bwd_bf16_kernel<D, false>), dim3((unsigned)nblk), dim3(256), 0, stream, q, k, v, g, lse,
                         Dws, acc, dK, dV, Tq, Tk, scale, cl2e, nkb, grad_f32);
  }
  if ((phases & FA_BWD_POST) && !grad_f32)
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)nfill), dim3(256), 0, stream, acc,
                       static_cast<uint16_t*>(dQ), nq);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int launch_bwd_bf16(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                    void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal,
                    int o_f32, int grad_f32, void* workspace, int phases, hipStream_t stream) {
  switch (d) {
    case 64: return bwd<64>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream);
    case 128: return bwd<128>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream);
    case 256: return bwd<256>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream);
    default: return FA_ERR_HEADDIM;
  }
}

}  // namespace fa
