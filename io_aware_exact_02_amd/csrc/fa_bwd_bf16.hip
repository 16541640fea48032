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
//   * Q_i and dO_i are read from HBM once (16-byte buffer loads, one block
//     ahead, into registers) and written to LDS twice: row-major for the
//     products that contract over the feature axis, and transposed (query
//     order permuted to match the MFMA k-slots) for the ones that contract
//     over queries.  lse_i (times log2 e) and D_i go to LDS as well.
//   * S = Q_i K_j^T on MFMA with one key per lane (Observation 1: the weights
//     are rebuilt as P = exp2(S * scale*log2e - lse*log2e)); only blocks that
//     cross the causal diagonal are masked.  Rows past Tq and keys past Tk
//     need no mask: their Q/dO or K/V rows read as zeros, so they add nothing.
//   * dV_j += P^T dO_i; dP = dO_i V_j^T; dS = P * (dP - D_i) (Observation 3);
//     dK_j += dS^T Q_i -- all on MFMA with P and dS taken from registers.
//   * dS (bf16) goes to LDS; after the block's one barrier the workgroup forms
//     dQ_i's contribution of all 128 keys, scale * dS K_j, and adds it to a
//     float32 accumulator in HBM with buffer atomics (rows past Tq are dropped
//     by the buffer range check).  The order in which different key blocks
//     add is not fixed, so dQ's last bits may vary between runs.
//   * Q/dO stages and the dS tile are double-buffered, so one barrier per
//     query block orders everything (the 256-wide heads use a single stage and
//     two barriers to stay within LDS).
// Before the sweep, a pre-pass writes D = rowsum(dO * O) (Observation 2) and
// clears the dQ accumulator; afterwards, if the caller wants bf16 dQ, a
// post-pass rounds the accumulator.
#include <type_traits>

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
  static constexpr int NST = D == 256 ? 1 : 2;  // Q/dO/dS stages
  static constexpr int NSTR = D + 8;            // row-major tiles (bf16 per row)
  static constexpr int TSTR = kBQ + 8;          // transposed Q/dO tiles: D rows of 32 queries
  static constexpr int KTSTR = kBKC + 8;        // transposed K tile: D rows of 128 keys
  static constexpr int SSTR = kBKC + 8;         // dS tile: 32 rows of 128 keys
  // byte offsets inside one stage
  static constexpr int Q_N = 0;
  static constexpr int Q_T = Q_N + kBQ * NSTR * 2;
  static constexpr int G_N = Q_T + D * TSTR * 2;
  static constexpr int G_T = G_N + kBQ * NSTR * 2;
  static constexpr int L_F = G_T + D * TSTR * 2;       // lse * log2 e [32]
  static constexpr int D_F = L_F + kBQ * 4;            // D [32]
  static constexpr int STAGE = D_F + kBQ * 4;
  static constexpr int S_OFF = NST * STAGE;            // dS tiles
  static constexpr int S_BYTES = kBQ * SSTR * 2;
  static constexpr int KT_OFF = S_OFF + NST * S_BYTES; // K^T of the key block
  static constexpr int BYTES = KT_OFF + D * KTSTR * 2;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NBLK = (kBQ / 8) * (D / 8);     // 8x8 blocks per tensor tile
  static_assert(STAGE % 16 == 0 && S_BYTES % 16 == 0, "LDS regions must stay 16-byte aligned");
  static_assert(2 * ((NBLK + 63) / 64) <= 4, "Q and dO staging waves fit in the workgroup");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float* __restrict__ lse, const float* __restrict__ Dr,
                     float* __restrict__ dQacc, void* __restrict__ dK, void* __restrict__ dV,
                     int Tq, int Tk, float scale, float cl2e, int nkb, int grad_f32) {
  using L = BwdLayout<D>;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  const int nblk = gridDim.x, wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int bh = lin / nkb;
  const int kblk = CAUSAL ? nkb - 1 - (lin % nkb) : (lin % nkb);   // causal: longest sweeps first
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hf = lane >> 5;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  const int k0 = kblk * kBKC;
  const int kw0 = k0 + wave * kKeysPerWave;
  const int mykey = kw0 + l32;

  const rsrc_t rq = make_rsrc(Q + qbase, (unsigned)Tq * D * 2u);
  const rsrc_t rg = make_rsrc(dO + qbase, (unsigned)Tq * D * 2u);
  const rsrc_t rk = make_rsrc(K + kbase, (unsigned)Tk * D * 2u);
  const rsrc_t rv = make_rsrc(V + kbase, (unsigned)Tk * D * 2u);
  const rsrc_t rl = make_rsrc(lse + (size_t)bh * Tq, (unsigned)Tq * 4u);
  const rsrc_t rd = make_rsrc(Dr + (size_t)bh * Tq, (unsigned)Tq * 4u);
  const rsrc_t racc = make_rsrc(dQacc + qbase, (unsigned)Tq * D * 4u);

  // K_j and V_j as B operands (column = key, k = features), held for the sweep.
  bf16x8 kf[L::NDS], vf[L::NDS];
#pragma unroll
  for (int ds = 0; ds < L::NDS; ++ds) {
    const unsigned off = ((unsigned)mykey * D + ds * 16 + 8 * hf) * 2u;
    kf[ds] = as_bf16x8(bload16(rk, off));
    vf[ds] = as_bf16x8(bload16(rv, off));
  }
  // K_j^T for the dQ product: 8x8 blocks (8 keys x 8 features) transposed into LDS
  for (int b = tid; b < (kBKC / 8) * (D / 8); b += 256) {
    const int kg = b % (kBKC / 8), dg = b / (kBKC / 8);
    u32x4 r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = bload16(rk, ((unsigned)(k0 + kg * 8 + i) * D + dg * 8) * 2u);
    char* kt = smem + L::KT_OFF + (dg * 8 * L::KTSTR + kg * 8) * 2;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x4 even, odd;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        even[p] = lo_lo(r[2 * p][w], r[2 * p + 1][w]);
        odd[p] = hi_hi(r[2 * p][w], r[2 * p + 1][w]);
      }
      st16(kt + (2 * w) * L::KTSTR * 2, even);
      st16(kt + (2 * w + 1) * L::KTSTR * 2, odd);
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
  // Whole waves stage one tensor each (so the buffer resource they load through
  // is wave-uniform): WPT waves per tensor, one 8x8 block (8 query rows x 8
  // features) per lane, features fastest across lanes so that a row-major store
  // covers whole rows.  The top 32 threads also fetch lse and D.  A tile index
  // past the sweep maps to row Tq, whose loads return zeros.
  constexpr int WPT = (L::NBLK + 63) / 64;
  const bool is_g = __builtin_amdgcn_readfirstlane(wave) >= WPT;
  const int tb = (wave % WPT) * 64 + lane;
  const bool tloader = wave < 2 * WPT && tb < L::NBLK;
  const rsrc_t rsrc_t_src = is_g ? rg : rq;
  const int dgq = tb % (D / 8), rg8 = tb / (D / 8);
  const int rt = rg8 >> 1, rh = rg8 & 1;
  auto trow = [&](int i) { return 16 * rt + 4 * rh + (i < 4 ? i : 4 + i); };
  const bool sloader = tid >= 256 - kBQ;
  const int srow = tid - (256 - kBQ);
  u32x4 stg[8];
  float sl = 0.f, sd = 0.f;
  auto first_row = [&](int it) { return it < nqt ? it * kBQ : Tq; };
  auto gload = [&](int r0) {
    if (tloader) {
#pragma unroll
      for (int i = 0; i < 8; ++i) stg[i] = bload16(rsrc_t_src, ((unsigned)(r0 + trow(i)) * D + dgq * 8) * 2u);
    }
    if (sloader) {
      sl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (r0 + srow) * 4, 0, 0));
      sd = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, (r0 + srow) * 4, 0, 0));
    }
  };
  auto lstore = [&](int st) {
    char* base = smem + st * L::STAGE;
    if (tloader) {
      char* N = base + (is_g ? L::G_N : L::Q_N);
      char* T = base + (is_g ? L::G_T : L::Q_T);
#pragma unroll
      for (int i = 0; i < 8; ++i) st16(N + (trow(i) * L::NSTR + dgq * 8) * 2, stg[i]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 even, odd;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          even[p] = lo_lo(stg[2 * p][w], stg[2 * p + 1][w]);
          odd[p] = hi_hi(stg[2 * p][w], stg[2 * p + 1][w]);
        }
        st16(T + ((dgq * 8 + 2 * w) * L::TSTR + 16 * rt + 8 * rh) * 2, even);
        st16(T + ((dgq * 8 + 2 * w + 1) * L::TSTR + 16 * rt + 8 * rh) * 2, odd);
      }
    }
    if (sloader) {
      reinterpret_cast<float*>(base + L::L_F)[srow] = sl * kLog2e;
      reinterpret_cast<float*>(base + L::D_F)[srow] = sd;
    }
  };

  gload(first_row(it0));
  lstore(0);
  wait_vmem_all();
  __syncthreads();

  // dQ atomics: lane = feature column, register r = query row 8(r/4)+4hf+r%4
  auto dq_product = [&](int r0, const char* ss) {
    for (int db = wave; db < L::NDB; db += kWavesB) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kBKC / 16; ++ks) {
        const bf16x8 a = as_bf16x8(ld16(ss + (l32 * L::SSTR + ks * 16 + 8 * hf) * 2));
        const bf16x8 b =
            as_bf16x8(ld16(smem + L::KT_OFF + ((db * 32 + l32) * L::KTSTR + ks * 16 + 8 * hf) * 2));
        acc = mfma32(a, b, acc);
      }
      // the whole byte offset goes in the vector offset, which the range check
      // covers: rows past Tq (whose contributions are zero anyway) are dropped
      const unsigned vo = ((unsigned)(r0 + 4 * hf) * D + db * 32 + l32) * 4u;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(scale * acc[r], racc,
                                                        vo + (unsigned)(8 * (r >> 2) + (r & 3)) * D * 4u, 0, 0);
    }
  };

  auto step = [&](int it, auto stage) {
    constexpr int ST = decltype(stage)::value;
    constexpr int NX = L::NST == 2 ? (ST ^ 1) : 0;    // stage the next block is written to
    const int r0 = it * kBQ;
    const char* sb_ = smem + ST * L::STAGE;
    char* ss = smem + L::S_OFF + ST * L::S_BYTES;
    gload(first_row(it + 1));

    // S = Q_i K_j^T and dP = dO_i V_j^T: lane = key, register r = query 8(r/4)+4hf+r%4
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int ds = 0; ds < L::NDS; ++ds) {
      const bf16x8 a = as_bf16x8(ld16(sb_ + L::Q_N + (l32 * L::NSTR + ds * 16 + 8 * hf) * 2));
      s = mfma32(a, kf[ds], s);
      const bf16x8 g = as_bf16x8(ld16(sb_ + L::G_N + (l32 * L::NSTR + ds * 16 + 8 * hf) * 2));
      dp = mfma32(g, vf[ds], dp);
    }
    const float* lsv = reinterpret_cast<const float*>(sb_ + L::L_F);
    const float* dsv_ = reinterpret_cast<const float*>(sb_ + L::D_F);
    float p[16], dsv[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int qr = 8 * g4 + 4 * hf;
      const f32x4 lv = *reinterpret_cast<const f32x4*>(lsv + qr);
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(dsv_ + qr);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g4 + e;
        p[r] = fast_exp2(__builtin_fmaf(s[r], cl2e, -lv[e]));
        dsv[r] = dp[r] - dv4[e];
      }
    }
    if (CAUSAL && r0 < kw0 + kKeysPerWave - 1) {       // block crosses this wave's diagonal
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (mykey > r0 + 8 * (r >> 2) + 4 * hf + (r & 3)) p[r] = 0.f;
    }
    bf16x8 pb[2], sbf[2];
    unsigned sw[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * t + 2 * e;
        a[e] = pack_bf16(p[r], p[r + 1]);
        b[e] = pack_bf16(p[r] * dsv[r], p[r + 1] * dsv[r + 1]);
        sw[4 * t + e] = b[e];
      }
      pb[t] = as_bf16x8(a);
      sbf[t] = as_bf16x8(b);
    }
    // dV_j += P^T dO_i ; dK_j += dS^T Q_i  (lane = feature column, register = key row)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < L::NDB; ++db) {
        const bf16x8 g = as_bf16x8(ld16(sb_ + L::G_T + ((db * 32 + l32) * L::TSTR + 16 * t + 8 * hf) * 2));
        dv[db] = mfma32(pb[t], g, dv[db]);
        const bf16x8 qq = as_bf16x8(ld16(sb_ + L::Q_T + ((db * 32 + l32) * L::TSTR + 16 * t + 8 * hf) * 2));
        dk[db] = mfma32(sbf[t], qq, dk[db]);
      }
    // dS -> LDS as [query][key]: word k holds queries qr and qr+1 of this lane's key
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 2 * k;
      const int qr = 8 * (r >> 2) + 4 * hf + (r & 3);
      uint16_t* dst = reinterpret_cast<uint16_t*>(ss) + qr * L::SSTR + wave * kKeysPerWave + l32;
      dst[0] = (uint16_t)(sw[k] & 0xffffu);
      dst[L::SSTR] = (uint16_t)(sw[k] >> 16);
    }
    if (L::NST == 2) {
      lstore(NX);
      wait_vmem_all();
      __syncthreads();
      dq_product(r0, ss);
    } else {
      wait_vmem_all();
      __syncthreads();
      dq_product(r0, ss);
      __syncthreads();
      lstore(0);
      __syncthreads();
    }
  };

  if (L::NST == 2) {
    for (int it = it0; it < nqt; it += 2) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < nqt) step(it + 1, std::integral_constant<int, 1>{});
    }
  } else {
    for (int it = it0; it < nqt; ++it) step(it, std::integral_constant<int, 0>{});
  }

  // dK_j = scale * dS^T Q, dV_j: lane = feature, register r = key 8(r/4)+4hf+r%4
  const unsigned gsz = grad_f32 ? 4u : 2u;
  const rsrc_t rdk = make_rsrc(static_cast<char*>(dK) + kbase * gsz, (unsigned)Tk * D * gsz);
  const rsrc_t rdv = make_rsrc(static_cast<char*>(dV) + kbase * gsz, (unsigned)Tk * D * gsz);
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      const unsigned idx = (unsigned)key * D + db * 32 + l32;
      const float gk = scale * dk[db][r], gv = dv[db][r];
      if (grad_f32) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, gk), rdk, idx * 4u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, gv), rdv, idx * 4u, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16(gk, 0.f) & 0xffffu), rdk, idx * 2u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16(gv, 0.f) & 0xffffu), rdv, idx * 2u, 0, 0);
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
