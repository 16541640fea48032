// Backward pass for bf16 inputs on gfx950 MFMA.
//
// [ZtF] = "FlashAttention", zerotofrontier.app textbook section 12.3,
// sections "The backward pass, derived" and "Which loop goes outside?".
//
// Every kernel here starts from the row terms D = rowsum(dO * O) that a
// pre-pass leaves in the workspace (Observation 2) and rebuilds the weights
// from lse as P = exp2(S * scale*log2e - lse*log2e) (Observation 1).
//
// Head widths 64 and 128: two sweeps, no atomics, each output summed in a
// fixed order.
//   * bwd_kv_kernel: one workgroup per block of 128 keys sweeps the query
//     blocks and writes dK_j and dV_j once.
//   * bwd_dq_kernel: one workgroup per block of 256 queries sweeps the key
//     blocks and writes dQ_i once.
// The split costs two extra tile products (S and dP are formed in both sweeps)
// but no dQ traffic beyond one write: adding each key block's share of dQ with
// float32 atomics would send Tk/128 partial sums per dQ element through the
// memory-side atomic units, which is slower on this part than recomputing.
//
// Head width 256 (bwd_bf16_w4_kernel): a single key-block sweep whose four
// waves each own 32 keys and keep K_j, V_j (as MFMA B operands) and the float32
// accumulators dK_j, dV_j in registers.  Per query block i:
//   * Q_i and dO_i are read from HBM once (16-byte buffer loads, one block
//     ahead, into registers) and written to LDS twice: row-major for the
//     products that contract over the feature axis, and transposed (query
//     order permuted to match the MFMA k-slots) for the ones that contract
//     over queries.  lse_i (times log2 e) and D_i go to LDS as well.
//   * S = Q_i K_j^T on MFMA with one key per lane; only blocks that cross the
//     causal diagonal are masked.  Rows past Tq and keys past Tk need no mask:
//     their Q/dO or K/V rows read as zeros, so they add nothing.
//   * dV_j += P^T dO_i; dP = dO_i V_j^T; dS = P * (dP - D_i) (Observation 3);
//     dK_j += dS^T Q_i -- all on MFMA with P and dS taken from registers.
//   * dS (bf16) goes to LDS; after the block's barrier the workgroup forms
//     dQ_i's contribution of all 128 keys, scale * dS K_j, and adds it to a
//     float32 accumulator in HBM with buffer atomics (rows past Tq are dropped
//     by the buffer range check).  The order in which different key blocks
//     add is not fixed, so dQ's last bits may vary between runs.  A pre-pass
//     clears the accumulator; a post-pass rounds it if the caller wants bf16.
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
void bwd_bf16_w4_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
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

// ---------------------------------------------------------------------------
// Row terms for the two sweeps below, stored negated so that they enter the
// sweeps without a subtraction: Dn_r = -(dO_r . O_r) ([ZtF] "The backward
// pass, derived", Observation 2) seeds the dP accumulator, so the MFMA returns
// dP - D directly; Ln_r = -lse_r log2 e is the addend of P's exponent.
// ---------------------------------------------------------------------------
template <int D, bool O_F32>
__global__ __launch_bounds__(256) void row_terms_kernel(const uint16_t* __restrict__ dO, const void* __restrict__ O,
                                                        const float* __restrict__ lse, float* __restrict__ Dn,
                                                        float* __restrict__ Ln, long long rows) {
  constexpr int G = D / 8;                 // lanes per row, 8 elements each
  constexpr int RPB = 256 / G;             // rows per block
  const long long r = (long long)blockIdx.x * RPB + threadIdx.x / G;
  const int j = threadIdx.x % G;
  float part = 0.f;
  if (r < rows) {
    const u32x4 g = ld16(dO + r * D + 8 * j);
    float o[8];
    if (O_F32) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(O) + r * D + 8 * j);
      const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(O) + r * D + 8 * j + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = a[e];
        o[4 + e] = b[e];
      }
    } else {
      const u32x4 w = ld16(static_cast<const uint16_t*>(O) + r * D + 8 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = __builtin_bit_cast(float, w[e] << 16);
        o[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      part = __builtin_fmaf(__builtin_bit_cast(float, g[e] << 16), o[2 * e], part);
      part = __builtin_fmaf(__builtin_bit_cast(float, g[e] & 0xffff0000u), o[2 * e + 1], part);
    }
  }
#pragma unroll
  for (int m = 1; m < G; m <<= 1) part += __shfl_xor(part, m, 64);
  if (r < rows && j == 0) {
    Dn[r] = -part;
    Ln[r] = -kLog2e * lse[r];
  }
}

// ---------------------------------------------------------------------------
// Key-block sweep for d = 64 and 128: dK_j and dV_j.
//
// One workgroup of eight waves per (128-key block, b, h), split by role so
// that each SIMD holds two waves of at most 256 registers and one wave's VALU
// or LDS waits are covered by the other's MFMA work:
//   * score waves 0-3 (32 keys each) keep their K_j and V_j fragments in
//     registers.  Per query tile: S = Q_i K_j^T and dP - D = dO_i V_j^T - D_i
//     on MFMA (the accumulator starts at -D), P = exp2(S c log2e - lse log2e)
//     and dS = P * (dP - D) ([ZtF] "The backward pass, derived", Observations
//     1-3), handed on through LDS as MFMA fragments (P^T and dS^T, one key per
//     lane).  lse and D of the next tile are fetched from HBM into registers
//     while the current tile is processed.
//   * gradient waves 4-7 (wave 4+w serves score wave w's keys) keep dV_j and
//     dK_j in float32 registers and trail the score waves by one query tile:
//     dV_j += P^T dO_i and dK_j += dS^T Q_i; they also stage Q_i and dO_i two
//     tiles ahead.
// One barrier per phase orders everything: the row-major stages and the
// fragment buffers alternate between two slots, the transposed Q/dO tiles
// between three (the gradient waves read tile i-1's while writing tile i+1's);
// the loops are unrolled so that every slot is a constant offset.
// Rows past Tq and keys past Tk need no masking: their Q/dO or K/V rows read
// as zeros, so they add nothing to the gradients that are stored.
// ---------------------------------------------------------------------------
template <int D>
struct KvLayout {
  static constexpr int NSTR = D + 8;            // row-major Q_i / dO_i (bf16 per row)
  static constexpr int TSTR = kBQ + 8;          // transposed tiles: D rows of 32 queries
  static constexpr int N_BYTES = kBQ * NSTR * 2;
  static constexpr int T_BYTES = D * TSTR * 2;
  static constexpr int Q_N = 0;                              // one stage: Q_i and dO_i row-major
  static constexpr int G_N = Q_N + N_BYTES;
  static constexpr int STAGE = G_N + N_BYTES;
  static constexpr int QT_OFF = 2 * STAGE;                   // Q_i^T, three slots
  static constexpr int GT_OFF = QT_OFF + 3 * T_BYTES;        // dO_i^T, three slots
  static constexpr int F_WAVE = 4 * 64 * 16;                 // P^T and dS^T fragments of one score wave
  static constexpr int F_BYTES = kWavesB * F_WAVE;
  static constexpr int F_OFF = GT_OFF + 3 * T_BYTES;         // two slots
  static constexpr int BYTES = F_OFF + 2 * F_BYTES;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int WPT = D / 64;                         // staging waves per tensor
  static constexpr int SW0 = 8 - 2 * WPT;                    // first staging wave
  static_assert(STAGE % 16 == 0 && T_BYTES % 16 == 0, "16-byte aligned regions");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Block-sparse sweeps ([ZtF] "Dropout, block-sparsity, and other real-kernel
// details"): the mask holds one byte per (128-query block, 128-key block).  A
// key block's workgroup visits only the query tiles whose block keeps it; each
// wave reads its mask column 64 blocks at a time as a bit word (a ballot, held
// in scalar registers) and walks the visible tiles with its own cursor.  Every
// wave derives the same sequence, so both roles pass the same number of
// barriers.
constexpr int kMaskBlock = 128;
constexpr int kTilesPerMaskRow = kMaskBlock / kBQ;
static_assert(kBKC == kMaskBlock, "one key-block workgroup per mask column");

template <int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(512) void bwd_kv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Ln, const float* __restrict__ Dn,
    void* __restrict__ dK, void* __restrict__ dV, int Tq, int Tk, float scale, float cl2e, int nkb, int grad_f32,
    const uint8_t* __restrict__ bmask, int H, long long mask_hstride, int nmk) {
  using L = KvLayout<D>;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  const int nblk = gridDim.x, wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int bh = lin / nkb;
  const int kblk = CAUSAL ? nkb - 1 - (lin % nkb) : (lin % nkb);   // causal: longest sweeps first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int wq = wave & 3;                      // key slice (score wave w and gradient wave 4+w)
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  const int k0 = kblk * kBKC;
  const int kw0 = k0 + wq * kKeysPerWave;
  const int mykey = kw0 + l32;

  const int nqt = (Tq + kBQ - 1) / kBQ;
  const int it0 = CAUSAL ? min(k0 / kBQ, nqt) : 0;
  // tile t covers query rows t kBQ ..; a tile past the sweep reads row Tq (zeros)
  auto tile_row = [&](int t) { return t < nqt ? t * kBQ : Tq; };

  // visible query tiles: all from it0 on, or (masked) those whose block bit is set
  const int nmq = (Tq + kMaskBlock - 1) / kMaskBlock;
  const int nvw = (nmq + 63) >> 6;
  const uint8_t* mcol = MASKED ? bmask + (long long)(bh % H) * mask_hstride + kblk : nullptr;
  // bit r of word w: query block 64w + r keeps this key block.  The word last
  // read is kept; a cursor moving forward reads again only every 64 blocks.
  int cw = -1;
  unsigned long long cbits = 0;
  auto word = [&](int w) {
    if (w != cw) {
      cw = w;
      cbits = mask_word(mcol, nmk, nmq, w, lane);
    }
    return cbits;
  };
  auto vis_row = [&](int r) { return ((word(r >> 6) >> (r & 63)) & 1ull) != 0; };
  auto next_row = [&](int r) {                  // first visible query block >= r, nmq if none
    int w = r >> 6;
    if (w >= nvw) return nmq;
    unsigned long long bits = word(w) & (~0ull << (r & 63));
    while (bits == 0) {
      if (++w >= nvw) return nmq;
      bits = word(w);
    }
    return w * 64 + (int)__builtin_ctzll(bits);
  };
  auto next_tile = [&](int t) {                 // first visible tile >= t (nqt if none)
    if constexpr (MASKED) {
      if (t >= nqt) return nqt;
      if (vis_row(t / kTilesPerMaskRow)) return t;
      const int r = next_row(t / kTilesPerMaskRow + 1);
      return r < nmq ? r * kTilesPerMaskRow : nqt;
    } else {
      return t;
    }
  };
  int n = nqt - it0;                            // query tiles in the sweep
  if constexpr (MASKED) {
    n = 0;
    if (it0 < nqt) {
      const int rlo = it0 / kTilesPerMaskRow;
      for (int w = rlo >> 6; w < nvw; ++w) {
        unsigned long long bits = word(w);
        if (w == (rlo >> 6)) bits &= ~0ull << (rlo & 63);
        n += __builtin_popcountll(bits);
      }
      n *= kTilesPerMaskRow;
      if (vis_row(rlo)) n -= it0 - rlo * kTilesPerMaskRow;          // first block starts at it0
      if (vis_row(nmq - 1)) n -= nmq * kTilesPerMaskRow - nqt;      // last block is ragged
    }
  }

  if (wave < 4) {
    // ============================ score waves ============================
    const rsrc_t rk = make_rsrc(K + kbase, (unsigned)Tk * D * 2u);
    const rsrc_t rv = make_rsrc(V + kbase, (unsigned)Tk * D * 2u);
    const rsrc_t rl = make_rsrc(Ln + (size_t)bh * Tq, (unsigned)Tq * 4u);
    const rsrc_t rd = make_rsrc(Dn + (size_t)bh * Tq, (unsigned)Tq * 4u);
    bf16x8 kf[L::NDS], vf[L::NDS];
#pragma unroll
    for (int ds = 0; ds < L::NDS; ++ds) {
      const unsigned off = ((unsigned)mykey * D + ds * 16 + 8 * hf) * 2u;
      kf[ds] = as_bf16x8(bload16(rk, off));
      vf[ds] = as_bf16x8(bload16(rv, off));
    }
    // -lse log2e and -D of the tile's queries in the accumulator order:
    // register r <-> query 8(r/4) + 4hf + r%4 (all lanes of a half alike)
    auto terms_load = [&](int t, f32x16& lt, f32x16& dt) {
      const int r0 = tile_row(t);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const unsigned off = (unsigned)(r0 + 8 * g4 + 4 * hf) * 4u;
        const f32x4 a = __builtin_bit_cast(f32x4, bload16(rl, off));
        const f32x4 b = __builtin_bit_cast(f32x4, bload16(rd, off));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lt[4 * g4 + e] = a[e];
          dt[4 * g4 + e] = b[e];
        }
      }
    };
    f32x16 lt0, dt0, lt1, dt1;
    int tc = next_tile(it0);                      // the tile of the next score step
    terms_load(tc, lt0, dt0);
    __syncthreads();

    // tile t in stage ST (the step's parity in the sweep); tn is the tile after it
    auto score_step = [&](int t, int tn, auto stage, const f32x16& lt, const f32x16& dt, f32x16& lt_n,
                          f32x16& dt_n) {
      constexpr int ST = decltype(stage)::value;
      terms_load(tn, lt_n, dt_n);
      const int r0 = t * kBQ;
      const char* sb_ = smem + ST * L::STAGE;
      // S = Q_i K_j^T and dP - D = dO_i V_j^T - D_i: lane = key, register r = query 8(r/4)+4hf+r%4
      f32x16 sacc, dp = dt;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      bf16x8 qa[L::NDS], ga[L::NDS];
#pragma unroll
      for (int ds = 0; ds < L::NDS; ++ds) {
        qa[ds] = as_bf16x8(ld16(sb_ + L::Q_N + (l32 * L::NSTR + ds * 16 + 8 * hf) * 2));
        ga[ds] = as_bf16x8(ld16(sb_ + L::G_N + (l32 * L::NSTR + ds * 16 + 8 * hf) * 2));
      }
#pragma unroll
      for (int ds = 0; ds < L::NDS; ++ds) {
        sacc = mfma32(qa[ds], kf[ds], sacc);
        dp = mfma32(ga[ds], vf[ds], dp);
      }
      sched_reads_ahead<2 * L::NDS>();
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(sacc[r], cl2e, lt[r]));
      if (CAUSAL && r0 < kw0 + kKeysPerWave - 1) {     // the tile crosses this wave's diagonal
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mykey > r0 + 8 * (r >> 2) + 4 * hf + (r & 3)) p[r] = 0.f;
      }
      // fragments for the gradient wave: [P^T t=0, P^T t=1, dS^T t=0, dS^T t=1], 1 KiB each
      char* fb = smem + L::F_OFF + ST * L::F_BYTES + wq * L::F_WAVE + lane * 16;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * t + 2 * e;
          a[e] = pack_bf16(p[r], p[r + 1]);
          b[e] = pack_bf16(p[r] * dp[r], p[r + 1] * dp[r + 1]);
        }
        st16(fb + t * 1024, a);
        st16(fb + (2 + t) * 1024, b);
      }
      __syncthreads();
    };
    for (int s = 0; s < n; s += 2) {
      int tn = next_tile(tc + 1);
      score_step(tc, tn, std::integral_constant<int, 0>{}, lt0, dt0, lt1, dt1);
      tc = tn;
      if (s + 1 < n) {
        tn = next_tile(tc + 1);
        score_step(tc, tn, std::integral_constant<int, 1>{}, lt1, dt1, lt0, dt0);
        tc = tn;
      }
    }
  } else {
    // =========================== gradient waves ==========================
    const rsrc_t rq = make_rsrc(Q + qbase, (unsigned)Tq * D * 2u);
    const rsrc_t rg = make_rsrc(dO + qbase, (unsigned)Tq * D * 2u);

    // Staging: WPT waves per tensor (Q, then dO); lane = 4 consecutive query rows
    // (quad qa) x 8 features (group fg), quads fastest across lanes.  A tile
    // index past the sweep maps to row Tq, whose loads return zeros.
    const bool stager = wave >= L::SW0;
    const bool is_g = wave >= L::SW0 + L::WPT;
    const int sidx = ((wave - L::SW0) % L::WPT) * 64 + lane;
    const int qa = sidx & 7, fg = sidx >> 3;
    const rsrc_t rsrc = is_g ? rg : rq;
    // transposed position of the quad: the middle quads of each 16 queries are
    // swapped, matching the query order of a fragment's MFMA k-slots
    const int tpos = 16 * (qa >> 2) + 4 * (((qa & 1) << 1) | ((qa >> 1) & 1));
    const int n_off = (is_g ? L::G_N : L::Q_N) + ((4 * qa) * L::NSTR + fg * 8) * 2;
    const int t_off = (is_g ? L::GT_OFF : L::QT_OFF) + ((fg * 8) * L::TSTR + tpos) * 2;
    u32x4 stg[4];
    auto gload = [&](int t) {
      if (stager) {
        const int r0 = tile_row(t);
#pragma unroll
        for (int i = 0; i < 4; ++i) stg[i] = bload16(rsrc, ((unsigned)(r0 + 4 * qa + i) * D + fg * 8) * 2u);
      }
    };
    auto lstore = [&](int slot2, int slot3) {     // slots s % 2 and s % 3 of the tile staged
      if (stager) {
        char* N = smem + slot2 * L::STAGE + n_off;
        char* T = smem + slot3 * L::T_BYTES + t_off;
#pragma unroll
        for (int i = 0; i < 4; ++i) st16(N + i * L::NSTR * 2, stg[i]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u32x2 ev = {lo_lo(stg[0][w], stg[1][w]), lo_lo(stg[2][w], stg[3][w])};
          const u32x2 od = {hi_hi(stg[0][w], stg[1][w]), hi_hi(stg[2][w], stg[3][w])};
          st8(T + (2 * w) * L::TSTR * 2, ev);
          st8(T + (2 * w + 1) * L::TSTR * 2, od);
        }
      }
    };

    f32x16 dk[L::NDB], dv[L::NDB];
#pragma unroll
    for (int db = 0; db < L::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[db][r] = 0.f;
        dv[db][r] = 0.f;
      }
    const int f_lane = L::F_OFF + wq * L::F_WAVE + lane * 16;
    const int t_lane = (l32 * L::TSTR + 8 * hf) * 2;

    // dV_j += P^T dO_i and dK_j += dS^T Q_i for the tile in slots (slot2, slot3):
    // lane = feature column, register = key row
    auto grad_step = [&](int slot2, int slot3) {
      const char* fb = smem + slot2 * L::F_BYTES + f_lane;
      const char* gt = smem + L::GT_OFF + slot3 * L::T_BYTES + t_lane;
      const char* qt = smem + L::QT_OFF + slot3 * L::T_BYTES + t_lane;
      bf16x8 pb[2], sbf[2], ga[2][L::NDB], qa[2][L::NDB];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        pb[t] = as_bf16x8(ld16(fb + t * 1024));
        sbf[t] = as_bf16x8(ld16(fb + (2 + t) * 1024));
#pragma unroll
        for (int db = 0; db < L::NDB; ++db) {
          const int toff = (db * 32 * L::TSTR + 16 * t) * 2;
          ga[t][db] = as_bf16x8(ld16(gt + toff));
          qa[t][db] = as_bf16x8(ld16(qt + toff));
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < L::NDB; ++db) {
          dv[db] = mfma32(pb[t], ga[t][db], dv[db]);
          dk[db] = mfma32(sbf[t], qa[t][db], dk[db]);
        }
      sched_reads_ahead<4 * L::NDB, 4 * L::NDB + 4>();
    };

    int tg = next_tile(it0);                         // the tile of the next fetch
    if (n > 0) {
      gload(tg);
      lstore(0, 0);
      tg = next_tile(tg + 1);
      if (n > 1) {
        gload(tg);
        tg = next_tile(tg + 1);
      }
    }
    __syncthreads();
    // phase p: gradients of sweep step p-1, stage step p+1, fetch step p+2.
    // m2 = p % 2 and m3 = p % 3 (wave-uniform counters) pick the slots.
    int m2 = 0, m3 = 0;
    for (int p = 0; p < n; ++p) {
      const int up3 = m3 == 2 ? 0 : m3 + 1;          // (p + 1) % 3
      const int dn3 = m3 == 0 ? 2 : m3 - 1;          // (p - 1) % 3
      if (p >= 1) grad_step(m2 ^ 1, dn3);
      if (p + 1 < n) lstore(m2 ^ 1, up3);
      if (p + 2 < n) {
        gload(tg);
        tg = next_tile(tg + 1);
      }
      __syncthreads();
      m2 ^= 1;
      m3 = up3;
    }
    // the last tile's gradients: its slots are ((n-1) % 2, (n-1) % 3)
    if (n > 0) grad_step(m2 ^ 1, m3 == 0 ? 2 : m3 - 1);

    // dK_j = scale * dS^T Q and dV_j: lane = feature, register r = key 8(r/4)+4hf+r%4
    const unsigned gsz = grad_f32 ? 4u : 2u;
    const rsrc_t rdk = make_rsrc(static_cast<char*>(dK) + kbase * gsz, (unsigned)Tk * D * gsz);
    const rsrc_t rdv = make_rsrc(static_cast<char*>(dV) + kbase * gsz, (unsigned)Tk * D * gsz);
#pragma unroll
    for (int db = 0; db < L::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned idx = (unsigned)(kw0 + 8 * (r >> 2) + 4 * hf + (r & 3)) * D + db * 32 + l32;
        const float gk = scale * dk[db][r];
        const float gv = dv[db][r];   // a scalar copy: bit-casting a vector element in place reads element 0
        if (grad_f32) {
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, gk), rdk, idx * 4u, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, gv), rdv, idx * 4u, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16(gk, 0.f) & 0xffffu), rdk, idx * 2u, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16(gv, 0.f) & 0xffffu), rdv, idx * 2u, 0, 0);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Query-block sweep for d = 64 and 128: dQ_i, in the other loop order ([ZtF]
// "Which loop goes outside?"), so that each dQ row is summed in registers by
// one wave and written once, with no atomics and a fixed summation order.
//
// One workgroup of eight waves per (256-query block, b, h); each wave owns 32
// query rows and keeps their Q and dO fragments (MFMA B operands), lse, D and
// the float32 dQ^T accumulator in registers for a sweep over key blocks of 64
// (causal: up to the block's last query; tiles a wave cannot see are skipped
// by that wave).  Per key block j:
//   * K_j and V_j go HBM -> LDS by buffer_load ... lds (rows XOR-swizzled by
//     16-byte chunk); K_j^T goes HBM -> registers -> LDS transposed, its key
//     order matching the k-slot order of the dS fragments below.
//   * S^T = K_j Q^T and dP^T - D = V_j dO^T - D on MFMA put one query per lane,
//     so lse and D are per-lane constants (-D seeds the accumulator):
//     P^T = exp2(S^T c log2e - lse log2e) and dS^T = P^T * (dP^T - D) ([ZtF]
//     "The backward pass, derived").
//   * dQ^T += K_j^T dS^T with dS^T rounded to bf16 straight from registers.
// Epilogue: dQ = scale * dQ~, once, in the gradient dtype.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqBR = 32 * kDqWaves;          // query rows per workgroup
constexpr int kDqBC = 64;                     // keys per block

template <int D>
struct DqLayout {
  static constexpr int BC = kDqBC;
  static constexpr int NC = D / 8;                     // 16-byte chunks per K/V row
  static constexpr int KST = BC * D * 2;               // K (or V) tile, swizzled rows, unpadded
  static constexpr int TSTR = BC + 8;                  // bf16 per K^T row (16-byte pad)
  static constexpr int TST = D * TSTR * 2;
  static constexpr int STAGE = 2 * KST + TST;
  static constexpr int BYTES = 2 * STAGE;
  static constexpr int NKB = BC / 32;
  static constexpr int NDB = D / 32;
  static constexpr int NDS = D / 16;
  static constexpr int KDMA = KST / 1024;              // 1 KiB DMA instructions per K (or V) tile
  static constexpr int KDMA_W = 2 * KDMA / kDqWaves;   // per wave: waves 0-3 load K, 4-7 load V
  static constexpr int NTB = (BC / 4) * (D / 8);       // 4 keys x 8 features blocks of K^T
  static_assert((2 * KDMA) % kDqWaves == 0 && KDMA % (kDqWaves / 2) == 0, "DMA split over the waves");
  static_assert(NTB <= 64 * kDqWaves, "one K^T block per thread at most");
  static_assert(NC == 8 || NC >= 16, "swizzle assumes 8 or >= 16 chunks per row");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
  static constexpr int k_off(int st) { return st * STAGE; }
  static constexpr int v_off(int st) { return st * STAGE + KST; }
  static constexpr int t_off(int st) { return st * STAGE + 2 * KST; }
};

// Chunk swizzle of row r of a K/V tile: with 16 or more chunks per row the 16
// rows a half-wave reads land on 16 distinct 16-byte bank groups; with 8 chunks
// (128-byte rows, two per 256-byte bank cycle) rows pair up by r >> 1.
template <int NC>
__device__ __forceinline__ int dq_swz(int r) { return NC >= 16 ? (r & 15) : ((r >> 1) & 7); }

// Block-sparse dQ sweep: the workgroup's 256 queries span two 128-query mask
// rows.  Both rows go into LDS bitmaps (bit c = key block c visible); the
// workgroup visits the key tiles that either row can see, and a wave computes
// only those its own row can see.
template <int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(512) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Ln, const float* __restrict__ Dn,
    void* __restrict__ dQ, int Tq, int Tk, float scale, float cl2e, int nqb, int grad_f32,
    const uint8_t* __restrict__ bmask, int H, long long mask_hstride, int nmk) {
  using L = DqLayout<D>;
  constexpr int BC = L::BC;
  static_assert(kMaskBlock % BC == 0 && kDqBR == 2 * kMaskBlock, "two mask rows, whole tiles per mask block");
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];

  const int nblk = gridDim.x, wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int bh = lin / nqb;
  const int qb = CAUSAL ? nqb - 1 - (lin % nqb) : (lin % nqb);    // causal: longest sweeps first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  const int q0 = qb * kDqBR;
  const int qw = q0 + wave * 32;
  const int myq = qw + lq;

  const rsrc_t rq = make_rsrc(Q + qbase, (unsigned)Tq * D * 2u);
  const rsrc_t rg = make_rsrc(dO + qbase, (unsigned)Tq * D * 2u);
  const rsrc_t rk = make_rsrc(K + kbase, (unsigned)Tk * D * 2u);
  const rsrc_t rv = make_rsrc(V + kbase, (unsigned)Tk * D * 2u);
  const rsrc_t rl = make_rsrc(Ln + (size_t)bh * Tq, (unsigned)Tq * 4u);
  const rsrc_t rd = make_rsrc(Dn + (size_t)bh * Tq, (unsigned)Tq * 4u);

  // Q and dO fragments (B operands): column = query, k = features
  bf16x8 qf[L::NDS], gf[L::NDS];
#pragma unroll
  for (int ds = 0; ds < L::NDS; ++ds) {
    const unsigned off = ((unsigned)myq * D + ds * 16 + 8 * hf) * 2u;
    qf[ds] = as_bf16x8(bload16(rq, off));
    gf[ds] = as_bf16x8(bload16(rg, off));
  }
  // -lse log2e and -D of this lane's query; -D seeds every dP^T accumulator
  const float lnq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, myq * 4, 0, 0));
  const float dnq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, myq * 4, 0, 0));
  f32x16 dseed;
#pragma unroll
  for (int r = 0; r < 16; ++r) dseed[r] = dnq;

  int ntile = (Tk + BC - 1) / BC;
  if (CAUSAL) ntile = min(ntile, (min(q0 + kDqBR, Tq) - 1) / BC + 1);

  // ---- K (waves 0-3) and V (waves 4-7): HBM -> LDS, swizzled
  const rsrc_t rkv = wave < kDqWaves / 2 ? rk : rv;
  auto kv_dma = [&](int k0, int st) {
#pragma unroll
    for (int i = 0; i < L::KDMA_W; ++i) {
      const int g = wave * L::KDMA_W + i;            // 0 .. 2 KDMA - 1; V's follow K's in the stage
      const int s = (g % L::KDMA) * 64 + lane;
      const int row = s / L::NC, cp = s % L::NC;
      const unsigned off = ((unsigned)(k0 + row) * D + (cp ^ dq_swz<L::NC>(row)) * 8) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rkv, (__attribute__((address_space(3))) void*)(smem + L::k_off(st) + g * 1024), 16, off, 0, 0, 0);
    }
  };
  // per-lane K/V read offset for k-step ds: chunk (2 ds + hf) ^ swz of row lq
  const int swz_l = dq_swz<L::NC>(lq);
  const int kbase_lane = lq * D * 2 + (((swz_l >> 1) << 5) | ((hf ^ (swz_l & 1)) << 4));

  // ---- K^T: HBM -> registers -> LDS transposed (4 keys x 8 features per thread)
  const bool t_loader = tid < L::NTB;
  const int kq = tid % (BC / 4), dg = tid / (BC / 4);
  const int kq3 = kq & 3;
  const int tpos = 16 * (kq >> 2) + 4 * (kq3 == 1 ? 2 : (kq3 == 2 ? 1 : kq3));
  u32x4 tst[4];
  auto t_load = [&](int k0) {
    if (t_loader) {
#pragma unroll
      for (int i = 0; i < 4; ++i) tst[i] = bload16(rk, ((unsigned)(k0 + 4 * kq + i) * D + dg * 8) * 2u);
    }
  };
  auto t_store = [&](int st) {
    if (t_loader) {
      char* base = smem + L::t_off(st) + (dg * 8 * L::TSTR + tpos) * 2;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 even = {lo_lo(tst[0][w], tst[1][w]), lo_lo(tst[2][w], tst[3][w])};
        const u32x2 odd = {hi_hi(tst[0][w], tst[1][w]), hi_hi(tst[2][w], tst[3][w])};
        st8(base + (2 * w) * L::TSTR * 2, even);
        st8(base + (2 * w + 1) * L::TSTR * 2, odd);
      }
    }
  };

  f32x16 dq[L::NDB];
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

  // ---- visible key tiles: bit c of word w of mask row a (b) = key block
  // 64w + c is kept for the first (second) 128 queries.  The words last read
  // are kept; a cursor moving forward reads again only every 64 key blocks.
  const int nvw = (nmk + 63) >> 6;
  const int mr = q0 / kMaskBlock;
  const bool has_b = mr + 1 < (Tq + kMaskBlock - 1) / kMaskBlock;
  const uint8_t* mrow = MASKED ? bmask + (long long)(bh % H) * mask_hstride + (long long)mr * nmk : nullptr;
  int cw = -1;
  unsigned long long ca = 0, cb = 0;
  auto words = [&](int w) {
    if (w != cw) {
      cw = w;
      ca = mask_word(mrow, 1, nmk, w, lane);
      cb = has_b ? mask_word(mrow + nmk, 1, nmk, w, lane) : 0ull;
    }
  };
  auto next_tile = [&](int j) {                       // first tile >= j either mask row sees, ntile if none
    if constexpr (MASKED) {
      if (j >= ntile) return ntile;
      const int c = j * BC / kMaskBlock;
      int w = c >> 6;
      words(w);
      unsigned long long bits = (ca | cb) & (~0ull << (c & 63));
      while (bits == 0) {
        if (++w >= nvw) return ntile;
        words(w);
        bits = ca | cb;
      }
      const int c2 = w * 64 + (int)__builtin_ctzll(bits);
      return c2 == c ? j : min(ntile, c2 * (kMaskBlock / BC));
    } else {
      return j;
    }
  };
  auto wave_sees = [&](int j) {                       // this wave's mask row sees tile j
    if constexpr (MASKED) {
      const int c = j * BC / kMaskBlock;
      words(c >> 6);
      return ((((wave >> 2) ? cb : ca) >> (c & 63)) & 1ull) != 0;
    } else {
      return true;
    }
  };

  auto first_row = [&](int j) { return j < ntile ? j * BC : Tk; };
  const int j0 = next_tile(0);
  kv_dma(first_row(j0), 0);
  t_load(first_row(j0));
  t_store(0);
  wait_vmem_all();
  __syncthreads();

  // tile j in stage ST (the step's parity in the sweep); jn is the tile after it
  auto step = [&](int j, int jn, auto stage) {
    constexpr int ST = decltype(stage)::value;
    // the mask test comes before the loads of block jn: a branch between those
    // loads and the reads of stage ST would make the compiler wait for the loads
    const bool sees = wave_sees(j);
    t_load(first_row(jn));
    kv_dma(first_row(jn), ST ^ 1);
    const int kt0 = j * BC;
    if ((!CAUSAL || kt0 <= qw + 31) && sees) {          // some key of the block is visible to this wave
      const bool edge = (CAUSAL && kt0 + BC - 1 > qw) || (kt0 + BC > Tk);
#pragma unroll
      for (int kb = 0; kb < L::NKB; ++kb) {
        // S^T and dP^T - D for 32 keys: register r = key kt0 + 32 kb + 8(r/4)+4hf+r%4, lane = query
        f32x16 s, dp = dseed;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        bf16x8 ka[L::NDS], va[L::NDS];
#pragma unroll
        for (int ds = 0; ds < L::NDS; ++ds) {
          const int off = kb * 32 * D * 2 + (kbase_lane ^ (ds << 5));
          ka[ds] = as_bf16x8(ld16(smem + L::k_off(ST) + off));
          va[ds] = as_bf16x8(ld16(smem + L::v_off(ST) + off));
        }
#pragma unroll
        for (int ds = 0; ds < L::NDS; ++ds) {
          s = mfma32(ka[ds], qf[ds], s);
          dp = mfma32(va[ds], gf[ds], dp);
        }
        sched_reads_ahead<2 * L::NDS>();
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(s[r], cl2e, lnq));
        if (edge) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= Tk || (CAUSAL && key > myq)) p[r] = 0.f;
          }
        }
        bf16x8 sf[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * t + 2 * e;
            w[e] = pack_bf16(p[r] * dp[r], p[r + 1] * dp[r + 1]);
          }
          sf[t] = as_bf16x8(w);
        }
        // dQ^T += K_j^T dS^T: lane = query column, register = feature row
        const char* ts = smem + L::t_off(ST);
        bf16x8 ta[2][L::NDB];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < L::NDB; ++db)
            ta[t][db] = as_bf16x8(ld16(ts + ((db * 32 + lq) * L::TSTR + kb * 32 + 16 * t + 8 * hf) * 2));
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < L::NDB; ++db) dq[db] = mfma32(ta[t][db], sf[t], dq[db]);
        if constexpr (2 * L::NDB >= 6) sched_reads_ahead<2 * L::NDB>();
      }
    }
    t_store(ST ^ 1);
    wait_vmem_all();
    __syncthreads();
  };

  if constexpr (MASKED) {
    for (int j = j0; j < ntile;) {
      int jn = next_tile(j + 1);
      step(j, jn, std::integral_constant<int, 0>{});
      j = jn;
      if (j >= ntile) break;
      jn = next_tile(j + 1);
      step(j, jn, std::integral_constant<int, 1>{});
      j = jn;
    }
  } else {
    for (int j = 0; j < ntile; j += 2) {
      step(j, j + 1, std::integral_constant<int, 0>{});
      if (j + 1 < ntile) step(j + 1, j + 2, std::integral_constant<int, 1>{});
    }
  }

  if (myq >= Tq) return;
  // dQ: lane = query, register 4g+e of block db = feature db*32 + 8g + 4hf + e
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * hf;
      const size_t off = qbase + (size_t)myq * D + d0;
      const float v0 = scale * dq[db][4 * g], v1 = scale * dq[db][4 * g + 1];
      const float v2 = scale * dq[db][4 * g + 2], v3 = scale * dq[db][4 * g + 3];
      if (grad_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(dQ) + off) = (f32x4){v0, v1, v2, v3};
      } else {
        const u32x2 w = {pack_bf16(v0, v1), pack_bf16(v2, v3)};
        st8(static_cast<uint16_t*>(dQ) + off, w);
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
        void* workspace, int phases, hipStream_t stream, const uint8_t* bmask, int mask_heads) {
  const long long rows = (long long)B * H * Tq;
  const long long nq = rows * D;
  const int nkb = (Tk + kBKC - 1) / kBKC;
  const long long nblk = (long long)nkb * B * H;
  const long long nfill = (nq + 1023) / 1024;
  const int nqb = (Tq + kDqBR - 1) / kDqBR;
  const long long nqblk = (long long)nqb * B * H;
  if (nblk > 0x7fffffffLL || nfill > 0x7fffffffLL || nqblk > 0x7fffffffLL) return FA_ERR_SHAPE;
  const float cl2e = scale * kLog2e;
  auto q = static_cast<const uint16_t*>(Q);
  auto k = static_cast<const uint16_t*>(K);
  auto v = static_cast<const uint16_t*>(V);
  auto g = static_cast<const uint16_t*>(dO);
  float* Dws = static_cast<float*>(workspace);
  // block mask [mask_heads][ceil(Tq/128)][ceil(Tk/128)]
  const int nmq = (Tq + kMaskBlock - 1) / kMaskBlock, nmk = (Tk + kMaskBlock - 1) / kMaskBlock;
  const long long mhs = mask_heads == 1 ? 0 : (long long)nmq * nmk;
  if constexpr (D == 256) {
    if (bmask) return FA_ERR_HEADDIM;
    // one key-block sweep that also adds dQ contributions into a float32 accumulator
    float* acc = grad_f32 ? static_cast<float*>(dQ) : Dws + bwd_rows_padded(rows);
    if (phases & FA_BWD_PRE) {
      hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)nfill), dim3(256), 0, stream, acc, nq);
      const int st = launch_rowdot_bf16(dO, O, o_f32, Dws, rows, D, stream);
      if (st != FA_OK) return st;
    }
    if (phases & FA_BWD_MAIN) {
      if (causal)
        hipLaunchKernelGGL((bwd_bf16_w4_kernel<D, true>), dim3((unsigned)nblk), dim3(256), 0, stream, q, k, v, g,
                           lse, Dws, acc, dK, dV, Tq, Tk, scale, cl2e, nkb, grad_f32);
      else
        hipLaunchKernelGGL((bwd_bf16_w4_kernel<D, false>), dim3((unsigned)nblk), dim3(256), 0, stream, q, k, v, g,
                           lse, Dws, acc, dK, dV, Tq, Tk, scale, cl2e, nkb, grad_f32);
    }
    if ((phases & FA_BWD_POST) && !grad_f32)
      hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)nfill), dim3(256), 0, stream, acc,
                         static_cast<uint16_t*>(dQ), nq);
  } else {
    // key-block sweep for dK, dV; query-block sweep for dQ; both read the
    // negated row terms Dn (workspace start) and Ln (after it)
    float* Dn = Dws;
    float* Ln = Dws + bwd_rows_padded(rows);
    if (phases & FA_BWD_PRE) {
      constexpr int RPB = 256 / (D / 8);
      const long long nrb = (rows + RPB - 1) / RPB;
      if (nrb > 0x7fffffffLL) return FA_ERR_SHAPE;
      if (o_f32)
        hipLaunchKernelGGL((row_terms_kernel<D, true>), dim3((unsigned)nrb), dim3(256), 0, stream, g, O, lse, Dn, Ln,
                           rows);
      else
        hipLaunchKernelGGL((row_terms_kernel<D, false>), dim3((unsigned)nrb), dim3(256), 0, stream, g, O, lse, Dn, Ln,
                           rows);
    }
    if (phases & FA_BWD_MAIN) {
      auto kv = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)nblk), dim3(512), 0, stream, q, k, v, g, Ln, Dn, dK, dV, Tq, Tk,
                           scale, cl2e, nkb, grad_f32, bmask, H, mhs, nmk);
      };
      if (bmask) {
        if (causal) kv(bwd_kv_kernel<D, true, true>);
        else kv(bwd_kv_kernel<D, false, true>);
      } else {
        if (causal) kv(bwd_kv_kernel<D, true, false>);
        else kv(bwd_kv_kernel<D, false, false>);
      }
    }
    if (phases & FA_BWD_POST) {
      auto dqk = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)nqblk), dim3(512), 0, stream, q, k, v, g, Ln, Dn, dQ, Tq, Tk,
                           scale, cl2e, nqb, grad_f32, bmask, H, mhs, nmk);
      };
      if (bmask) {
        if (causal) dqk(bwd_dq_kernel<D, true, true>);
        else dqk(bwd_dq_kernel<D, false, true>);
      } else {
        if (causal) dqk(bwd_dq_kernel<D, true, false>);
        else dqk(bwd_dq_kernel<D, false, false>);
      }
    }
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int launch_bwd_bf16(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                    void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal,
                    int o_f32, int grad_f32, void* workspace, int phases, hipStream_t stream, const uint8_t* bmask,
                    int mask_heads) {
  switch (d) {
    case 64: return bwd<64>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream, bmask, mask_heads);
    case 128: return bwd<128>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream, bmask, mask_heads);
    case 256: return bwd<256>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream, bmask, mask_heads);
    default: return FA_ERR_HEADDIM;
  }
}

}  // namespace fa
