// Split-key forward for few query rows (decoding), bf16 inputs on gfx950.
//
// [Atlas] "The version ladder: FA1 -> FA2 -> FA3" and [ZtF] "What it bought,
// measured": with one or a few query rows per head the query-block grid of the
// ordinary forward has too few workgroups to keep the GPU busy, so the key
// axis is split as well and the partial results are merged afterwards with the
// online-softmax rule ([Atlas] "Online softmax: the trick that makes tiling
// exact"): partial (m_p, l_p, O~_p) combine as m = max m_p,
// l = sum_p 2^(m_p - m) l_p, O = sum_p 2^(m_p - m) O~_p / l.
//
// Pass 1 (decode_partial_kernel): one workgroup of four waves per (32-query
// block, b, h, key chunk); wave w takes every fourth 32-key tile of the chunk
// and keeps its own running maximum, sums and O~ for the block's 32 query rows
// (one query per lane, as in the forward).  K rows go straight from HBM into
// MFMA fragments (S^T = K Q^T: the A operand is one key row per lane); V goes
// HBM -> registers -> the wave's own LDS region transposed, for O~^T += V^T P~^T.
// No workgroup barrier: each wave works alone, and with eight waves per CU the
// loads of one cover the arithmetic of the others.  The pass is bound by the
// HBM read of K and V.  Each wave writes its partial (O~, m, l, l~) to the
// workspace; the same lazy rescale and rounded-weight normaliser as the
// forward are used (m in scale*log2(e) units, l~ = sum of the bf16 weights).
// Pass 2 (decode_merge_kernel): one group of d/4 lanes per query row merges
// the partials and writes O (bf16 or float32) and lse.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecRows = 32;          // query rows per workgroup
constexpr int kDecKeys = 32;          // keys per tile
constexpr float kDecSlack = 8.0f;     // lazy rescale threshold, log2 units

template <int D>
struct DecLayout {
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int VSTR = kDecKeys + 8;            // bf16 per V^T row (16-byte pad)
  static constexpr int VWAVE = D * VSTR * 2;           // one wave's V^T tile
  static constexpr int BYTES = kDecWaves * VWAVE;
  static constexpr int NVB = (kDecKeys / 4) * (D / 8); // 4 keys x 8 features blocks per tile
  static constexpr int VPL = NVB / 64;                 // blocks per lane
  static_assert(NVB % 64 == 0, "whole blocks per lane");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void decode_partial_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                           const uint16_t* __restrict__ V, float* __restrict__ part_o,
                           float* __restrict__ part_s, int Tq, int Tk, float cl2e, int nqb, int nsplit,
                           int chunk_tiles, long long rows_total) {
  using L = DecLayout<D>;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  const int split = blockIdx.x % nsplit;
  const int qb = (blockIdx.x / nsplit) % nqb;
  const int bh = blockIdx.x / (nsplit * nqb);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  const int q0 = qb * kDecRows;
  const int myq = q0 + lq;
  char* vt = smem + wave * L::VWAVE;

  const rsrc_t rq = make_rsrc(Q + qbase, (unsigned)Tq * D * 2u);
  const rsrc_t rk = make_rsrc(K + kbase, (unsigned)Tk * D * 2u);
  const rsrc_t rv = make_rsrc(V + kbase, (unsigned)Tk * D * 2u);

  bf16x8 qf[L::NDS];
#pragma unroll
  for (int ds = 0; ds < L::NDS; ++ds) qf[ds] = as_bf16x8(bload16(rq, ((unsigned)myq * D + ds * 16 + 8 * hf) * 2u));

  // tiles of this chunk; causal: none past the block's last row (top-left)
  int t_end = min((split + 1) * chunk_tiles, (Tk + kDecKeys - 1) / kDecKeys);
  if (CAUSAL) t_end = min(t_end, (min(q0 + kDecRows, Tq) - 1) / kDecKeys + 1);
  const int t_beg = split * chunk_tiles + wave;

  // V block b of the tile for this lane: 4 keys (quad kq) x 8 features (group dg)
  int vkq[L::VPL], vdg[L::VPL], vpos[L::VPL];
#pragma unroll
  for (int i = 0; i < L::VPL; ++i) {
    const int blk = lane + 64 * i;
    vkq[i] = blk % (kDecKeys / 4);
    vdg[i] = blk / (kDecKeys / 4);
    const int k3 = vkq[i] & 3;
    // the middle quads of each 16 keys are swapped so the 8 keys an MFMA k-slot
    // half needs are contiguous (the k-slot order of the P~ fragments)
    vpos[i] = 16 * (vkq[i] >> 2) + 4 * (k3 == 1 ? 2 : (k3 == 2 ? 1 : k3));
  }

  f32x16 o[L::NDB];
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_ref = -INFINITY, l_part = 0.f, lr_part = 0.f;

  for (int t = t_beg; t < t_end; t += kDecWaves) {
    const int kt0 = t * kDecKeys;
    bf16x8 kfr[L::NDS];
#pragma unroll
    for (int ds = 0; ds < L::NDS; ++ds)
      kfr[ds] = as_bf16x8(bload16(rk, ((unsigned)(kt0 + lq) * D + ds * 16 + 8 * hf) * 2u));
    u32x4 vr[L::VPL][4];
#pragma unroll
    for (int i = 0; i < L::VPL; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) vr[i][e] = bload16(rv, ((unsigned)(kt0 + 4 * vkq[i] + e) * D + vdg[i] * 8) * 2u);

    // S^T = K Q^T: register r = key kt0 + 8(r/4)+4hf+r%4, lane = query
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < L::NDS; ++ds) s = mfma32(kfr[ds], qf[ds], s);

    // V^T into this wave's LDS region (wave-private: LDS operations of one wave
    // complete in order, so no barrier is needed)
#pragma unroll
    for (int i = 0; i < L::VPL; ++i) {
      char* base = vt + (vdg[i] * 8 * L::VSTR + vpos[i]) * 2;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 even = {lo_lo(vr[i][0][w], vr[i][1][w]), lo_lo(vr[i][2][w], vr[i][3][w])};
        const u32x2 odd = {hi_hi(vr[i][0][w], vr[i][1][w]), hi_hi(vr[i][2][w], vr[i][3][w])};
        st8(base + (2 * w) * L::VSTR * 2, even);
        st8(base + (2 * w + 1) * L::VSTR * 2, odd);
      }
    }

    if (kt0 + kDecKeys > Tk || (CAUSAL && kt0 + kDecKeys - 1 > q0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key >= Tk || (CAUSAL && key > myq)) s[r] = -INFINITY;
      }
    }
    float mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) mq[q] = fmaxf(fmaxf(s[4 * q], s[4 * q + 1]), fmaxf(s[4 * q + 2], s[4 * q + 3]));
    float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    mx = half_swap_max(mx) * cl2e;
    const bool grow = mx > m_ref + kDecSlack;
    if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
      const float alpha = grow ? fast_exp2(m_ref - mx) : 1.f;
      if (grow) m_ref = mx;
#pragma unroll
      for (int db = 0; db < L::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      l_part *= alpha;
      lr_part *= alpha;
    }
    const float mneg = (m_ref == -INFINITY) ? 0.f : -m_ref;
    bf16x8 pf[2];
    float ps[4] = {0.f, 0.f, 0.f, 0.f}, prs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * tt + 2 * e;
        const float p0 = fast_exp2(__builtin_fmaf(s[r], cl2e, mneg));
        const float p1 = fast_exp2(__builtin_fmaf(s[r + 1], cl2e, mneg));
        ps[e] += p0 + p1;
        w[e] = pack_bf16(p0, p1);
        prs[e] = add_bf16_pair(w[e], prs[e]);
      }
      pf[tt] = as_bf16x8(w);
    }
    l_part += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    lr_part += (prs[0] + prs[1]) + (prs[2] + prs[3]);
    // O~^T += V^T P~^T: lane = query column, register = feature row
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < L::NDB; ++db) {
        const bf16x8 a = as_bf16x8(ld16(vt + ((db * 32 + lq) * L::VSTR + 16 * tt + 8 * hf) * 2));
        o[db] = mfma32(a, pf[tt], o[db]);
      }
  }

  // partial of this wave: O~ rows (float32), then (m, l, l~) per row
  const float l_tot = half_swap_sum(l_part);
  const float lr_tot = half_swap_sum(lr_part);
  if (myq >= Tq) return;
  const long long p = (long long)split * kDecWaves + wave;
  const long long row = (long long)bh * Tq + myq;
  float* po = part_o + (p * rows_total + row) * D;
#pragma unroll
  for (int db = 0; db < L::NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 w = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
      *reinterpret_cast<f32x4*>(po + db * 32 + 8 * g + 4 * hf) = w;
    }
  if (hf == 0) {
    const f32x4 st = {m_ref, l_tot, lr_tot, 0.f};
    *reinterpret_cast<f32x4*>(part_s + (p * rows_total + row) * 4) = st;
  }
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_s, void* __restrict__ O,
                                                           float* __restrict__ lse, int nparts,
                                                           long long rows_total) {
  constexpr int G = D / 4;                         // lanes per row, 4 features each
  constexpr int RPB = 256 / G;                     // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / G;
  const int j = threadIdx.x % G;
  if (row >= rows_total) return;
  float m = -INFINITY;
  for (int p = 0; p < nparts; ++p) m = fmaxf(m, part_s[((long long)p * rows_total + row) * 4]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f, lr = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const f32x4 st = *reinterpret_cast<const f32x4*>(part_s + ((long long)p * rows_total + row) * 4);
    if (st[0] == -INFINITY) continue;                // a partial that saw no key
    const float a = fast_exp2(st[0] - m);
    l = __builtin_fmaf(a, st[1], l);
    lr = __builtin_fmaf(a, st[2], lr);
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + ((long long)p * rows_total + row) * D + 4 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(a, v[e], acc[e]);
  }
  const float inv = 1.f / lr;
  if (OUT_F32) {
    const f32x4 w = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(static_cast<float*>(O) + row * D + 4 * j) = w;
  } else {
    const u32x2 w = {pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
    st8(static_cast<uint16_t*>(O) + row * D + 4 * j, w);
  }
  if (j == 0) lse[row] = (m + log2f(l)) * kLn2;
}

template <int D>
int decode(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq, int Tk,
           float scale, int causal, int out_f32, int nsplit, void* workspace, hipStream_t stream) {
  const int nqb = (Tq + kDecRows - 1) / kDecRows;
  const int ntiles = (Tk + kDecKeys - 1) / kDecKeys;
  const int chunk_tiles = (ntiles + nsplit - 1) / nsplit;
  const long long rows = (long long)B * H * Tq;
  const long long nblk = (long long)B * H * nqb * nsplit;
  const long long nmerge = (rows + 256 / (D / 4) - 1) / (256 / (D / 4));
  if (nblk > 0x7fffffffLL || nmerge > 0x7fffffffLL) return FA_ERR_SHAPE;
  const long long nparts = (long long)nsplit * kDecWaves;
  float* part_o = static_cast<float*>(workspace);
  float* part_s = part_o + nparts * rows * D;
  const float cl2e = scale * kLog2e;
  auto q = static_cast<const uint16_t*>(Q);
  auto k = static_cast<const uint16_t*>(K);
  auto v = static_cast<const uint16_t*>(V);
  if (causal)
    hipLaunchKernelGGL((decode_partial_kernel<D, true>), dim3((unsigned)nblk), dim3(256), 0, stream, q, k, v, part_o,
                       part_s, Tq, Tk, cl2e, nqb, nsplit, chunk_tiles, rows);
  else
    hipLaunchKernelGGL((decode_partial_kernel<D, false>), dim3((unsigned)nblk), dim3(256), 0, stream, q, k, v,
                       part_o, part_s, Tq, Tk, cl2e, nqb, nsplit, chunk_tiles, rows);
  if (out_f32)
    hipLaunchKernelGGL((decode_merge_kernel<D, true>), dim3((unsigned)nmerge), dim3(256), 0, stream, part_o, part_s, O,
                       lse, (int)nparts, rows);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, false>), dim3((unsigned)nmerge), dim3(256), 0, stream, part_o, part_s,
                       O, lse, (int)nparts, rows);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int splitkv_parts(int B, int H, int Tq, int Tk, int nsplit) {
  const int ntiles = (Tk + kDecKeys - 1) / kDecKeys;
  if (nsplit <= 0) {
    // enough workgroups for two rounds over the 256 CUs, but chunks of at least
    // eight tiles per wave
    const long long base = (long long)B * H * ((Tq + kDecRows - 1) / kDecRows);
    long long want = (512 + base - 1) / base;
    const long long cap = (ntiles + 8 * kDecWaves - 1) / (8 * kDecWaves);
    nsplit = (int)(want < 1 ? 1 : (want > cap ? (cap < 1 ? 1 : cap) : want));
  }
  if (nsplit > ntiles) nsplit = ntiles;
  return nsplit;
}

int launch_decode_bf16(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq,
                       int Tk, int d, float scale, int causal, int out_f32, int nsplit, void* workspace,
                       hipStream_t stream) {
  switch (d) {
    case 64: return decode<64>(Q, K, V, O, lse, B, H, Tq, Tk, scale, causal, out_f32, nsplit, workspace, stream);
    case 128: return decode<128>(Q, K, V, O, lse, B, H, Tq, Tk, scale, causal, out_f32, nsplit, workspace, stream);
    default: return FA_ERR_HEADDIM;
  }
}

}  // namespace fa
