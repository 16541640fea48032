// Forward pass for bf16 inputs on gfx950 MFMA, FlashAttention-2 order.
//
// [ZtF] = "FlashAttention", zerotofrontier.app textbook section 12.3.
//
// One workgroup owns a block of BR = 128 query rows of one (batch, head) and
// makes one sweep over the key/value blocks ([ZtF] "The forward pass"); each
// of its four waves owns 32 query rows.  Per key block of BC keys:
//   * K_j and V_j are read from HBM with 16-byte coalesced loads into
//     registers one block ahead, then written to a double-buffered LDS stage.
//     V is transposed on the way (8x8 bf16 blocks in registers) so that every
//     MFMA operand read below is one conflict-free ds_read_b128.
//   * S^T = K_j Q_i^T on 32x32x16 bf16 MFMA with Q_i held in registers.  The
//     transposed product puts one query row per lane (and its other half in
//     lane ^ 32), so the row maximum and row sum are register reductions plus
//     one v_permlane32_swap.
//   * Masking only where a tile crosses the causal diagonal or the key tail
//     ([ZtF] "The causal mask, and the tiles you never visit": tiles above the
//     diagonal are never loaded -- the sweep stops at the block's last query).
//   * P~ = exp2(S * scale*log2(e) - m) with the hardware exp2; the running sum
//     l and output O~ are rescaled by exp2(m_old - m_new) ([ZtF] step 2.5)
//     only when the running maximum grew by more than 8 (log2 units): between
//     rescales both keep the same reference, so the final O~/l is unchanged
//     and P~ stays <= 2^8.
//   * O~^T += V_j^T P~^T on MFMA, P~ taken straight from the S registers
//     (rounded to bf16).
// Epilogue: O = O~/l rounded to bf16, lse = ln2 * (m + log2 l) ([ZtF] step 3).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D> struct FwdTile;
template <> struct FwdTile<64>  { static constexpr int BC = 128; };
template <> struct FwdTile<128> { static constexpr int BC = 64; };
template <> struct FwdTile<256> { static constexpr int BC = 32; };

constexpr int kWaves = 4;
constexpr int kBR = 32 * kWaves;          // query rows per workgroup
constexpr float kRescaleSlack = 8.0f;     // log2 units

template <int D>
struct FwdLayout {
  static constexpr int BC = FwdTile<D>::BC;
  static constexpr int KSTR = D + 8;        // bf16 per K row in LDS (16 B pad)
  static constexpr int VSTR = BC + 8;       // bf16 per V^T row in LDS (16 B pad)
  static constexpr int KELEMS = BC * KSTR;
  static constexpr int VELEMS = D * VSTR;
  static constexpr int STAGE = KELEMS + VELEMS;
  static constexpr int NKB = BC / 32;       // 32-key MFMA blocks per tile
  static constexpr int NDB = D / 32;        // 32-wide output blocks
  static constexpr int NDS = D / 16;        // k-steps of the QK^T product
  // Every tile holds BC*D = 8192 elements of K and of V: 128 threads move V as
  // 8x8 blocks, the other 128 move K as 8 chunks of 16 bytes each.
  static_assert(BC * D == 8192, "tile loader assumes 8192-element tiles");
};

// Position of key x (0..15) of a 16-key group inside its V^T row: the middle
// two quads are swapped so that the 8 keys one MFMA k-slot half needs
// (quads {h, h+2}) are contiguous.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2)))
void fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ lse, int Tq, int Tk, float cl2e, int nqb) {
  using L = FwdLayout<D>;
  constexpr int BC = L::BC;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

  // Workgroup -> (head, query block).  Consecutive workgroup ids go to
  // different XCDs round-robin; remapping gives each XCD a contiguous range of
  // logical blocks, so one head's query blocks (which share K and V) run on
  // the same L2.  Within a head the longest causal blocks start first.
  const int nblk = gridDim.x;
  const int wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int bh = lin / nqb;
  const int qb = nqb - 1 - (lin % nqb);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, hf = lane >> 5;
  const size_t qbase = (size_t)bh * Tq * D;
  const size_t kbase = (size_t)bh * Tk * D;
  const int q0 = qb * kBR;
  const int qw = q0 + wave * 32;
  const int myq = qw + lq;
  const bool wave_active = qw < Tq;

  // Q_i fragments (B operand of S^T = K Q^T): column = query, k = features.
  bf16x8 qf[L::NDS];
#pragma unroll
  for (int ds = 0; ds < L::NDS; ++ds) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (myq < Tq) v = ld16(Q + qbase + (size_t)myq * D + ds * 16 + 8 * hf);
    qf[ds] = as_bf16x8(v);
  }

  int ntile = (Tk + BC - 1) / BC;
  if (CAUSAL) {
    const int last_q = min(q0 + kBR, Tq) - 1;
    ntile = min(ntile, last_q / BC + 1);
  }
  const int last_q_wave = min(qw + 31, Tq - 1);

  // ---- global -> register staging of one K/V tile ----
  u32x4 stg[8];
  const bool v_loader = tid < 128;
  const int lt = v_loader ? tid : tid - 128;
  // V loader: 8x8 block (key group gk, feature group dg)
  const int gk = lt % (BC / 8), dg = lt / (BC / 8);
  const int vt = gk >> 1, vh = gk & 1;
  auto vkey = [&](int i) { return 16 * vt + 4 * vh + (i < 4 ? i : 4 + i); };

  auto gload = [&](int j) {
    const int k0 = j * BC;
    if (v_loader) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = k0 + vkey(i);
        stg[i] = (key < Tk) ? ld16(V + kbase + (size_t)key * D + dg * 8) : (u32x4){0u, 0u, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = lt + 128 * i;
        const int row = c / (D / 8), col8 = c % (D / 8);
        const int key = k0 + row;
        stg[i] = (key < Tk) ? ld16(K + kbase + (size_t)key * D + col8 * 8) : (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* Ks = smem + buf * L::STAGE;
    uint16_t* Vs = Ks + L::KELEMS;
    if (v_loader) {
      // column c of the 8x8 block -> V^T row dg*8+c, positions 16*vt + 8*vh .. +7
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 even, odd;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          even[p] = lo_lo(stg[2 * p][w], stg[2 * p + 1][w]);
          odd[p] = hi_hi(stg[2 * p][w], stg[2 * p + 1][w]);
        }
        st16(Vs + (dg * 8 + 2 * w) * L::VSTR + 16 * vt + 8 * vh, even);
        st16(Vs + (dg * 8 + 2 * w + 1) * L::VSTR + 16 * vt + 8 * vh, odd);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = lt + 128 * i;
        const int row = c / (D / 8), col8 = c % (D / 8);
        st16(Ks + row * L::KSTR + col8 * 8, stg[i]);
      }
    }
  };

  f32x16 o[L::NDB];
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_ref = -INFINITY;   // reference maximum, scale*log2(e) units
  float l_part = 0.f;        // this lane's share of the running sum

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < ntile; ++j) {
    if (j + 1 < ntile) gload(j + 1);
    const int k0 = j * BC;
    const bool compute = wave_active && (!CAUSAL || k0 <= last_q_wave);
    if (compute) {
      const uint16_t* Ks = smem + (j & 1) * L::STAGE;
      const uint16_t* Vs = Ks + L::KELEMS;
      // S^T = K_j Q_i^T
      f32x16 s[L::NKB];
#pragma unroll
      for (int kb = 0; kb < L::NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ds = 0; ds < L::NDS; ++ds) {
          const bf16x8 a = as_bf16x8(ld16(Ks + (kb * 32 + lq) * L::KSTR + ds * 16 + 8 * hf));
          s[kb] = mfma32(a, qf[ds], s[kb]);
        }
      }
      // mask: causal diagonal tiles and the key tail only
      const bool need_mask = (CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > Tk);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= Tk || (CAUSAL && key > myq)) s[kb][r] = -INFINITY;
          }
      }
      // row maximum of the tile
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_ref, mx * cl2e);
      const bool grow = m_new > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
        const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
        if (grow) m_ref = m_new;
#pragma unroll
        for (int db = 0; db < L::NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        l_part *= alpha;
      }
      const float mneg = (m_ref == -INFINITY) ? 0.f : -m_ref;
      // P~ = exp2(S * scale*log2e - m), packed to bf16 B operands
      bf16x8 pf[L::NKB][2];
#pragma unroll
      for (int kb = 0; kb < L::NKB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(__builtin_fmaf(s[kb][r], cl2e, mneg));
          l_part += p[r];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack_bf16(p[8 * t + 2 * e], p[8 * t + 2 * e + 1]);
          pf[kb][t] = as_bf16x8(w);
        }
      }
      // O~^T += V_j^T P~^T
#pragma unroll
      for (int db = 0; db < L::NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 a = as_bf16x8(ld16(Vs + (db * 32 + lq) * L::VSTR + kb * 32 + 16 * t + 8 * hf));
            o[db] = mfma32(a, pf[kb][t], o[db]);
          }
    }
    if (j + 1 < ntile) lstore((j + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = half_swap_sum(l_part);
  if (myq >= Tq) return;
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * hf;
      u32x2 w;
      w[0] = pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
      w[1] = pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      st8(O + qbase + (size_t)myq * D + d0, w);
    }
  if (hf == 0) lse[(size_t)bh * Tq + myq] = (m_ref + __log2f(l_tot)) * kLn2;
}

template <int D>
int launch(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq,
           int Tk, float scale, int causal, hipStream_t stream) {
  const int nqb = (Tq + kBR - 1) / kBR;
  const long long nblk = (long long)nqb * B * H;
  if (nblk > 0x7fffffffLL) return FA_ERR_SHAPE;
  const float cl2e = scale * kLog2e;
  dim3 grid((unsigned)nblk), block(256);
  auto q = static_cast<const uint16_t*>(Q);
  auto k = static_cast<const uint16_t*>(K);
  auto v = static_cast<const uint16_t*>(V);
  auto o = static_cast<uint16_t*>(O);
  if (causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, true>), grid, block, 0, stream, q, k, v, o, lse, Tq, Tk, cl2e, nqb);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, false>), grid, block, 0, stream, q, k, v, o, lse, Tq, Tk, cl2e, nqb);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int launch_fwd_bf16(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H,
                    int Tq, int Tk, int d, float scale, int causal, hipStream_t stream) {
  switch (d) {
    case 64: return launch<64>(Q, K, V, O, lse, B, H, Tq, Tk, scale, causal, stream);
    case 128: return launch<128>(Q, K, V, O, lse, B, H, Tq, Tk, scale, causal, stream);
    case 256: return launch<256>(Q, K, V, O, lse, B, H, Tq, Tk, scale, causal, stream);
    default: return FA_ERR_HEADDIM;
  }
}

}  // namespace fa
