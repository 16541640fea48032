// Forward pass for bf16 inputs on gfx950 MFMA, FlashAttention-2 order.
//
// [ZtF] = "FlashAttention", zerotofrontier.app textbook section 12.3.
//
// fwd_bf16_kernel (d = 64 and 128): one workgroup owns a block of 128 query
// rows of one (batch, head) and makes one sweep over the key/value blocks
// ([ZtF] "The forward pass"); each of its four waves owns 32 query rows, held
// as MFMA B operands in registers.  d = 256 runs fwd_split_kernel, further
// down, in two wave roles.  Under a
// plain causal mask a workgroup runs two blocks in turn, a short and a long one,
// so that all workgroups sweep about the same number of key blocks.
//
// Data movement per key block j of BC keys:
//   * K_j goes HBM -> LDS with buffer_load ... lds (no registers, no VALU):
//     lane l of a load lands at LDS base + 16 l, so the 16-byte chunks of a K
//     row are placed XOR-swizzled by row, which makes the MFMA operand reads
//     below conflict-free without padding.  Rows past Tk read as zeros.
//   * V_j goes HBM -> LDS the same way, row-major with its own chunk swizzle;
//     the PV product reads its transposed operand (one feature per lane, 8
//     keys) with two transposing 8-byte LDS reads per MFMA, conflict-free.
// Products (32x32x16 bf16 MFMA, float32 accumulation):
//   * S^T = K_j Q^T puts one query row per lane (its other half in lane ^ 32):
//     the row maximum and sum are register reductions plus a v_permlane32_swap.
//   * O~^T += V_j^T P~^T with P~ taken straight from the S registers.
// Softmax ([ZtF] steps 2.3-2.5), in scale*log2(e) units with the hardware
// exp2: P~ = exp2(S c - m) against a reference maximum m that is moved (and O~
// and the sums rescaled by exp2(m_old - m_new)) only when a row's maximum has
// grown past it by more than 8; in between, the same reference holds for
// numerator and denominator, so the result is unchanged and P~ <= 2^8.  The
// row maximum is formed only on tiles where some lane's share of the tile's
// row sum exceeds 2^8: below that, no weight can, so no score passed the
// reference by more than the slack.
// Two running sums: the unrounded one gives lse; O~ is divided by the sum of
// the bf16-rounded weights the PV product actually used, which cancels the
// rounding of a row's dominant weight to first order.
// Masking only on tiles that cross the causal diagonal or the key tail; tiles
// above the diagonal are never loaded ([ZtF] "The causal mask, and the tiles
// you never visit": the sweep stops at the block's last query).
//
// One barrier per block: block j's S, softmax and PV run while K_{j+1} and
// V_{j+1} are in flight from HBM into the other LDS stage.  On gfx950 the MFMA
// and vector-ALU work of a SIMD overlap only in part, within a wave and across
// its two waves, so the softmax is kept to as few vector instructions per score
// as possible.
// Epilogue ([ZtF] step 3): O = O~/l (bf16 or float32), lse = ln2 (m + log2 l).
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D> struct FwdCfg;
template <> struct FwdCfg<64>  { static constexpr int BC = 64; static constexpr int WAVES_PER_EU = 2; };
template <> struct FwdCfg<128> { static constexpr int BC = 64; static constexpr int WAVES_PER_EU = 2; };

constexpr int kWaves = 4;
constexpr int kBR = 32 * kWaves;     // query rows per workgroup
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr float kMaxWeight = 256.0f;   // 2^kRescaleSlack

template <int D>
struct FwdLayout {
  static constexpr int BC = FwdCfg<D>::BC;
  static constexpr int NC = D / 8;                   // 16-byte chunks per K / V row
  static constexpr int RB = D * 2;                   // bytes per row
  static constexpr int KST = BC * RB;                // bytes per K (or V) stage (unpadded, swizzled)
  static constexpr int BYTES = 4 * KST;
  static constexpr int NKB = BC / 32;                // 32-key MFMA blocks per tile
  static constexpr int NDB = D / 32;                 // 32-feature output blocks
  static constexpr int NDS = D / 16;                 // k-steps of the QK^T product
  static constexpr int KDMA = KST / 1024;            // 1 KB LDS-load instructions per K (or V) tile
  static constexpr int KDMA_W = KDMA / kWaves;       // ... per wave
  static_assert(KDMA % kWaves == 0, "K tile must split evenly over the waves");
  static_assert(NC == 8 || NC >= 16, "swizzle assumes 8 or >= 16 chunks per row");
  static constexpr int K_OFF = 0, V_OFF = KST;      // within a stage
};

// Chunk swizzle of K row r: with 16 or more chunks per row the 16 rows a
// half-wave reads land on 16 distinct 16-byte bank groups; with 8 chunks
// (128-byte rows, two per 256-byte bank cycle) rows pair up by r >> 1.
template <int NC>
__device__ __forceinline__ int kswz(int r) { return NC >= 16 ? (r & 15) : ((r >> 1) & 7); }

// Chunk swizzle of V row r, for the transposing reads: a half-wave reads four
// consecutive rows x four chunks (8 bytes per lane), and XOR-ing the chunk's
// bits 2-3 with the row's position among the four (bit 2 with the row pair for
// 128-byte rows) puts those 32 reads on 64 distinct banks.  The swizzle only
// moves chunk bits >= 2, so a feature block's offset is a XOR with (db << 6).
template <int NC>
__device__ __forceinline__ int vswz(int r) { return NC == 8 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); }

// BAND (1 sliding window, 2 documents): each query row r sees the keys
// lo(r) .. hi(r) of a Band, both non-decreasing in r.  Key blocks outside the block's band are never visited; elements are masked
// only on tiles that cross a band edge of some row of the wave.
template <int D, bool CAUSAL, bool OUT_F32, bool MASKED, int BAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FwdCfg<D>::WAVES_PER_EU)))
void fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, void* __restrict__ O,
                     float* __restrict__ lse, int Tq, int Tk, float cl2e, int nqb,
                     const uint8_t* __restrict__ bmask, int H, long long mask_hstride, int nmk, int wl, int wr,
                     const int* __restrict__ cu, int nd, int bcausal) {
  using L = FwdLayout<D>;
  constexpr int BC = L::BC;
  static_assert(D == 64 || D == 128, "d = 256 runs fwd_split_kernel");
  // One LDS array per pipeline stage: accesses to distinct arrays carry distinct
  // alias scopes, which lets the compiler see that reads of one stage do not
  // touch the DMA in flight into the other (it would wait for the DMA otherwise).
  __shared__ __attribute__((aligned(1024))) char stage0[L::BYTES / 2];
  __shared__ __attribute__((aligned(1024))) char stage1[L::BYTES / 2];
  auto stage_ptr = [&](auto st) -> char* {
    if constexpr (decltype(st)::value == 0) return stage0;
    else return stage1;
  };

  // Workgroup -> (head, query blocks).  Consecutive workgroup ids go to
  // different XCDs round-robin; remapping gives each XCD a contiguous range of
  // logical blocks, so one head's query blocks (which share K and V) run on
  // the same L2.
  // Plain causal: workgroup p of a head runs query block nqb-1-p, then block p,
  // so every workgroup sweeps about the same number of key tiles.  With one
  // block each, lengths range from 1 to nqb blocks' worth, and the dispatcher
  // leaves CUs with a free slot idle for tens of microseconds at a time.
  // Otherwise one block per workgroup, the longest causal blocks first.
  constexpr bool PAIRED = CAUSAL && !MASKED && BAND == 0;
  const int nblk = gridDim.x;
  const int wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int npb = PAIRED ? (nqb + 1) / 2 : nqb;     // workgroups per head
  const int bh = lin / npb;
  const int pidx = lin % npb;
  const int npass = (PAIRED && 2 * pidx + 1 < nqb) ? 2 : 1;

  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, hf = lane >> 5;
  const size_t qbase = (size_t)bh * Tq * D;
  const size_t kbase = (size_t)bh * Tk * D;
  // Every wave runs every block's barriers; the early exits below only skip the
  // epilogue.  A block's last step ends on a barrier after all its LDS reads, so
  // the next block's first DMA cannot overwrite a tile still in use.
  for (int pass = 0; pass < npass; ++pass) {
    // the long block first: a head's workgroups start their long sweeps together
    // and share each K/V tile in L2; the staggered sweeps are the short ones
    const int qb = (npass == 2 && pass == 1) ? pidx : nqb - 1 - pidx;
    const int q0 = qb * kBR;
    const int qw = q0 + wave * 32;
    const int myq = qw + lq;

    // Buffer resource over the head's Q: rows past Tq read as zeros.
    const rsrc_t rq = make_rsrc(Q + qbase, (unsigned)Tq * D * 2u);

    // Q fragments (B operand of S^T = K Q^T): column = query, k = features.
    bf16x8 qf[L::NDS];
#pragma unroll
    for (int ds = 0; ds < L::NDS; ++ds)
      qf[ds] = as_bf16x8(bload16(rq, ((unsigned)myq * D + ds * 16 + 8 * hf) * 2u));

    int ntile = (Tk + BC - 1) / BC;
    if (CAUSAL) ntile = min(ntile, (min(q0 + kBR, Tq) - 1) / BC + 1);
    int jfirst = 0;                     // first key block any row of the block can see
    // BAND: this lane's keys klo .. khi; over the wave's rows the largest lo and
    // the smallest hi (a tile between them needs no element mask)
    int klo = 0, khi = 0, w_lo = 0, w_hi = 0;
    if constexpr (BAND != 0) {
      const Band<BAND> band{wl, wr, cu, nd, bcausal};
      band.keys(myq, klo, khi);
      w_lo = band.lo(qw + 31);
      w_hi = band.hi(qw);
      const int b_hi = band.hi(min(q0 + kBR, Tq) - 1);
      ntile = min(ntile, b_hi < 0 ? 0 : b_hi / BC + 1);
      jfirst = max(0, band.lo(q0)) / BC;
    }

    // ---- K and V: HBM -> LDS, swizzled.  Wave w issues DMA instructions g = w*KDMA_W + i;
    // lane l of instruction g moves chunk s = 64 g + l of the tile: row s / NC, stored
    // chunk s % NC, which holds source chunk (s % NC) ^ swizzle(row).  The lane offsets
    // within a tile do not change between tiles; the tile's start goes into a buffer
    // resource over rows k0 .. Tk-1 (scalar work only), so rows past Tk -- and whole
    // tiles past the end -- read as zeros, and the wave index (a scalar) gives the
    // LDS destination without vector instructions.
    unsigned koff[L::KDMA_W], voff[L::KDMA_W];
#pragma unroll
    for (int i = 0; i < L::KDMA_W; ++i) {
      const int s = (wave * L::KDMA_W + i) * 64 + lane;
      const int row = s / L::NC, cp = s % L::NC;
      koff[i] = (unsigned)(row * D + (cp ^ kswz<L::NC>(row)) * 8) * 2u;
      voff[i] = (unsigned)(row * D + (cp ^ vswz<L::NC>(row)) * 8) * 2u;
    }
    auto tile_dma = [&](const uint16_t* base, int k0, char* dst, const unsigned* off) {
      const int rows = Tk - k0;
      const rsrc_t r = make_rsrc(base + kbase + (size_t)(k0 < Tk ? k0 : 0) * D, rows > 0 ? (unsigned)rows * D * 2u : 0u);
#pragma unroll
      for (int i = 0; i < L::KDMA_W; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(dst + (wave * L::KDMA_W + i) * 1024), 16, off[i], 0, 0, 0);
    };
    auto k_dma = [&](int k0, char* kst) { tile_dma(K, k0, kst, koff); };
    auto v_dma = [&](int k0, char* vst) { tile_dma(V, k0, vst, voff); };
    // Per-lane K read offset (bytes, relative to a stage and a 32-key block) for
    // k-step ds: chunk (2 ds + hf) ^ swz of row lq.  The XOR only touches bits 5..7
    // of kbase_lane (rows are >= 128 bytes), so each k-step is kbase_lane ^ (ds << 5).
    const int kswz_l = kswz<L::NC>(lq);
    const int kbase_lane = lq * D * 2 + (((kswz_l >> 1) << 5) | ((hf ^ (kswz_l & 1)) << 4));

    // ---- V^T operand (A of O^T += V^T P^T): lane l, row feature 32 db + l % 32,
    // elements = keys 16t + 4hf + 0..3 and 16t + 8 + 4hf + 0..3 of key block kb,
    // the order of the P fragment's k-slots.  Each comes from one transposing read
    // in which lane 16g + 4e + j addresses key row 4(g/2) + e and features
    // 16(g%2) + 4j .. +3 (plus 32kb + 16t, and 8 for the second read).
    const int vg = lane >> 4, vi = lane & 15;
    const int vrow = 4 * (vg >> 1) + (vi >> 2);
    const int vc0 = 2 * (vg & 1) + ((vi & 3) >> 1);
    const int vlane = vrow * L::RB + ((vc0 ^ vswz<L::NC>(vrow)) << 4) + 8 * (vi & 1);

    f32x16 o[L::NDB];
#pragma unroll
    for (int db = 0; db < L::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_ref = -INFINITY;   // reference maximum, scale*log2(e) units
    float l_part = 0.f;        // this lane's share of the sum of the weights
    float lr_part = 0.f;       // ... and of the bf16-rounded weights

    auto s_product = [&](f32x16 (&s)[L::NKB], const char* kst) {
#pragma unroll
      for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      bf16x8 ka[L::NDS][L::NKB];
#pragma unroll
      for (int ds = 0; ds < L::NDS; ++ds)
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
          ka[ds][kb] = as_bf16x8(ld16(kst + kb * 32 * D * 2 + (kbase_lane ^ (ds << 5))));
#pragma unroll
      for (int ds = 0; ds < L::NDS; ++ds)
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb) s[kb] = mfma32(ka[ds][kb], qf[ds], s[kb]);
      sched_reads_ahead<L::NDS * L::NKB>();
    };
    auto mask_tile = [&](f32x16 (&s)[L::NKB], int j) {
      const int k0 = j * BC;
      if constexpr (BAND != 0) {
        // inside the band of every row of the wave: no element mask needed
        if (k0 >= w_lo && k0 + BC - 1 <= w_hi && k0 + BC <= Tk) return;
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= Tk || key < klo || key > khi) s[kb][r] = -INFINITY;
          }
        return;
      }
      if ((CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > Tk)) {
        // key k0 + c of register (kb, r) is masked iff c > lim, where c = 32 kb +
        // 8 (r / 4) + r % 4 + 4 hf and lim is the lane's last visible key - k0; the
        // sign of lim - c selects -inf by a bitfield insert (no per-score condition
        // registers)
        int lim = Tk - 1 - k0;
        if (CAUSAL) lim = min(lim, myq - k0);
        lim -= 4 * hf;
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned m = (unsigned)((lim - (kb * 32 + 8 * (r >> 2) + (r & 3))) >> 31);   // all ones iff masked
            const float x = s[kb][r];   // a scalar copy: bit_cast of a vector element in place reads element 0
            s[kb][r] = __builtin_bit_cast(float, (m & 0xff800000u) | (~m & __builtin_bit_cast(unsigned, x)));
          }
      }
    };

    // Key blocks the sweep visits: all of them, or (block mask, [ZtF] "Dropout,
    // block-sparsity, and other real-kernel details") only those whose 128-key
    // mask block is kept for this 128-row block; next_tile(j) is the first
    // visited block at or after j (ntile when none is left).  The mask row is
    // read 64 blocks at a time as a bit word held in scalar registers.
    static_assert(kBR == 128 && 128 % BC == 0, "one mask row per query block, whole key blocks per mask block");
    const uint8_t* mrow = MASKED ? bmask + (bh % H) * mask_hstride + (long long)qb * nmk : nullptr;
    const int nvw = (nmk + 63) >> 6;
    int cw = -1;
    unsigned long long cbits = 0;
    auto word = [&](int w) {
      if (w != cw) {
        cw = w;
        cbits = mask_word(mrow, 1, nmk, w, lane);
      }
      return cbits;
    };
    auto next_tile = [&](int j) {
      if constexpr (MASKED) {
        if (j >= ntile) return ntile;
        const int c = (j * BC) >> 7;
        int w = c >> 6;
        unsigned long long bits = word(w) & (~0ull << (c & 63));
        while (bits == 0) {
          if (++w >= nvw) return ntile;
          bits = word(w);
        }
        const int c2 = w * 64 + (int)__builtin_ctzll(bits);
        return c2 == c ? j : min(ntile, (c2 << 7) / BC);
      } else {
        return j;
      }
    };

    // ---- prologue: the first visited K and V block into LDS stage 0
    // A block index past the sweep maps to row Tk: its loads return zeros and
    // move no data, so the steps below need no branches around their loads.
    auto first_row = [&](int j) { return j < ntile ? j * BC : Tk; };
    const int j0 = next_tile(jfirst);
    k_dma(first_row(j0), stage_ptr(std::integral_constant<int, 0>{}) + L::K_OFF);
    v_dma(first_row(j0), stage_ptr(std::integral_constant<int, 0>{}) + L::V_OFF);
    wait_vmem_all();
    __syncthreads();

    auto step = [&](int j, int jn, auto stage) {
      constexpr int ST = decltype(stage)::value;        // position of block j in the sweep, mod 2
      // the next visited block jn in flight, straight into the other LDS stage
      char* const cur = stage_ptr(std::integral_constant<int, ST>{});
      char* const nxt = stage_ptr(std::integral_constant<int, ST ^ 1>{});
      k_dma(first_row(jn), nxt + L::K_OFF);
      v_dma(first_row(jn), nxt + L::V_OFF);
      f32x16 s[L::NKB];
      s_product(s, cur + L::K_OFF);
      // V^T operands of the PV product.  At d = 128 they are read here, so that
      // their latency hides behind the softmax (with the softmax's fast path below,
      // 255 registers and no spill); at d = 64 after it.
      const char* vs = cur + L::V_OFF;
      bf16x8 va[L::NKB][2][L::NDB];
      auto read_va = [&]() {
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int db = 0; db < L::NDB; ++db) {
              const char* p = vs + (32 * kb + 16 * t) * L::RB + (vlane ^ (db << 6));
              const u32x2 lo = ld8_tr(p), hi = ld8_tr(p + 8 * L::RB);
              va[kb][t][db] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
      };
      if constexpr (D == 128) read_va();
      mask_tile(s, j);
      // P~ rounded to bf16 for the PV product, and this lane's shares of both row sums
      bf16x8 pf[L::NKB][2];
      float ps[4], prs[4];
      auto weights = [&](float mneg) {
        // -0 + x is x for every x, so the first additions into ps fold away
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ps[e] = -0.f;
          prs[e] = 0.f;
        }
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * t + 2 * e;
              const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], cl2e, mneg));
              const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], cl2e, mneg));
              ps[e] += p0 + p1;
              w[e] = pack_bf16(p0, p1);
              prs[e] = add_bf16_pair(w[e], prs[e]);
            }
            pf[kb][t] = as_bf16x8(w);
          }
      };
      // Fast path: with the reference maximum kept, a lane's share of the tile's
      // row sum bounds each weight it holds, so shares of at most 2^slack on every
      // lane mean that no score passed the reference by more than the slack: no
      // rescale is due and the row maximum is not needed.  Otherwise (a row's
      // first block, a grown maximum, overflow, NaN) it is formed and the weights
      // redone, with the same decisions as without the fast path.
      bool need_max = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0ull;
      if (!need_max) {
        weights(-m_ref);
        const float share = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        need_max = __builtin_amdgcn_ballot_w64(!(share <= kMaxWeight)) != 0ull;
      }
      if (need_max) {
        // row maximum as shallow trees of independent partial results: long
        // chains of dependent vector ops leave the wave stalled
        float mq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // chain q folds s[kb][4q .. 4q+3] for every kb, two new values per max3
          float m = max3f(s[0][4 * q], s[0][4 * q + 1], s[0][4 * q + 2]);
          float pend = s[0][4 * q + 3];
          bool has = true;
#pragma unroll
          for (int kb = 1; kb < L::NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (has) m = max3f(m, pend, s[kb][4 * q + e]);
              else pend = s[kb][4 * q + e];
              has = !has;
            }
          mq[q] = has ? max2f(m, pend) : m;
        }
        float mx = max2f(max3f(mq[0], mq[1], mq[2]), mq[3]);
        mx = half_swap_max(mx) * cl2e;
        const bool grow = mx > m_ref + kRescaleSlack;     // never true for a row with no visible key yet
        if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
          const float alpha = grow ? fast_exp2(m_ref - mx) : 1.f;   // 0 on a row's first block
          if (grow) m_ref = mx;
#pragma unroll
          for (int db = 0; db < L::NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
          l_part *= alpha;
          lr_part *= alpha;
        }
        weights((m_ref == -INFINITY) ? 0.f : -m_ref);
      }
      l_part += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      lr_part += (prs[0] + prs[1]) + (prs[2] + prs[3]);
      // O~^T += V_j^T P~_j^T (independent accumulators back to back)
      if constexpr (D != 128) read_va();
#pragma unroll
      for (int kb = 0; kb < L::NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < L::NDB; ++db) o[db] = mfma32(va[kb][t][db], pf[kb][t], o[db]);
      if constexpr (D != 128) sched_reads_ahead<L::NKB * 2 * L::NDB, 2 * L::NKB * 2 * L::NDB>();
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
      for (int j = j0; j < ntile; j += 2) {
        step(j, j + 1, std::integral_constant<int, 0>{});
        if (j + 1 < ntile) step(j + 1, j + 2, std::integral_constant<int, 1>{});
      }
    }

    if (qw >= Tq) continue;
    const float l_tot = half_swap_sum(l_part);
    const float lr_tot = half_swap_sum(lr_part);
    if (myq >= Tq) continue;
    // a row that sees no key (possible only under a block mask or a band) gets O = 0, lse = -inf
    const float inv = (!(MASKED || BAND != 0) || lr_tot > 0.f) ? 1.f / lr_tot : 0.f;
#pragma unroll
    for (int db = 0; db < L::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hf;
        const size_t off = qbase + (size_t)myq * D + d0;
        if (OUT_F32) {
          const f32x4 w = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(static_cast<float*>(O) + off) = w;
        } else {
          u32x2 w;
          w[0] = pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
          w[1] = pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
          st8(static_cast<uint16_t*>(O) + off, w);
        }
      }
    if (hf == 0)
      lse[(size_t)bh * Tq + myq] = (!(MASKED || BAND != 0) || l_tot > 0.f) ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Forward for d = 256 in two roles (fwd_split_kernel), under every mask form:
// full, causal, block mask, sliding window and packed documents.
//
// With one wave per 32-row slice, the Q fragments (64 registers per lane), the
// O~ accumulator (128) and the V^T operands (64) oversubscribe a wave's
// registers; and since the lazy rescale multiplies O~ with vector
// instructions, the compiler keeps O~ in VGPRs and copies it into AGPRs and
// back around every PV product (some 300 moves per 32 MFMAs).  Here a
// workgroup of eight waves covers 128 rows, two waves per slice and per SIMD:
//   * score wave w (0-3) keeps slice w's Q fragments and the softmax state,
//     forms S^T = K_j Q^T, masks, forms P~ (the same fast and slow paths as
//     fwd_bf16_kernel) and hands P~ on through LDS as two MFMA fragments, with
//     the rescale factor of any row whose reference maximum moved;
//   * PV wave 4+w keeps slice w's O~^T and trails its score wave by one key
//     block: it applies a rescale when one was handed on, then O~^T +=
//     V_j^T P~_j^T with V_j^T by transposing reads.  The PV waves also issue the
//     copies of K and V (inline assembly, two blocks ahead, ring of four stages).
// At the end the score wave writes lse and hands 1/l~ to the PV wave, which
// writes O.  Each slice's arithmetic, masks and the order of its sums are those
// of one wave of fwd_bf16_kernel with 32-key blocks; against the one-role form
// at d = 256 that it replaced, the results were the same bits.
// ---------------------------------------------------------------------------
template <int D>
struct FwdSplitLayout {
  static constexpr int BC = 32;
  static constexpr int NC = D / 8;
  static constexpr int RB = D * 2;
  static constexpr int KST = BC * RB;                  // K (or V) tile, swizzled rows
  static constexpr int STAGE = 2 * KST;
  static constexpr int NSTAGE = 4;
  static constexpr int F_OFF = NSTAGE * STAGE;         // per slot and score wave: P~ (2 KiB), alpha (256 B), flag
  static constexpr int F_WAVE = 2048 + 256 + 256;
  static constexpr int F_SLOT = 4 * F_WAVE;
  static constexpr int E_OFF = F_OFF + 2 * F_SLOT;     // 1/l~ per lane of each score wave, at the end
  static constexpr int BYTES = E_OFF + 4 * 256;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int COPIES = STAGE / 1024 / 4;      // 1 KiB copies per PV wave and block
  static constexpr int K_OFF = 0, V_OFF = KST;
  static_assert(NC >= 16 && STAGE % 1024 == 0 && COPIES <= 15, "layout");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int D, bool CAUSAL, bool OUT_F32, bool MASKED, int BAND>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                      const uint16_t* __restrict__ V, void* __restrict__ O, float* __restrict__ lse, int Tq, int Tk,
                      float cl2e, int nqb, const uint8_t* __restrict__ bmask, int H, long long mask_hstride, int nmk,
                      int wl, int wr, const int* __restrict__ cu, int nd, int bcausal) {
  using L = FwdSplitLayout<D>;
  constexpr int BC = L::BC;
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
  auto stage_ptr = [&](int st) { return smem + st * L::STAGE; };

  constexpr bool PAIRED = CAUSAL && !MASKED && BAND == 0;
  const int nblk = gridDim.x;
  const int wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int npb = PAIRED ? (nqb + 1) / 2 : nqb;     // workgroups per head
  const int bh = lin / npb;
  const int pidx = lin % npb;
  const int npass = (PAIRED && 2 * pidx + 1 < nqb) ? 2 : 1;

  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, hf = lane >> 5;
  const int ws = wave & 3;                          // row slice (score wave ws, PV wave 4+ws)
  const size_t qbase = (size_t)bh * Tq * D;
  const size_t kbase = (size_t)bh * Tk * D;
  for (int pass = 0; pass < npass; ++pass) {
    if (pass > 0) {
      wait_lds_all();
      barrier_keep_vmem();
    }
    const int qb = (npass == 2 && pass == 1) ? pidx : nqb - 1 - pidx;
    const int q0 = qb * kBR;
    const int qw = q0 + ws * 32;
    const int myq = qw + lq;
    int ntile = (Tk + BC - 1) / BC;
    if (CAUSAL) ntile = min(ntile, (min(q0 + kBR, Tq) - 1) / BC + 1);
    int jfirst = 0;                     // first key block any row of the block can see
    // BAND: this lane's keys klo .. khi; over the slice's rows the largest lo and
    // the smallest hi (a tile between them needs no element mask)
    int klo = 0, khi = 0, w_lo = 0, w_hi = 0;
    if constexpr (BAND != 0) {
      const Band<BAND> band{wl, wr, cu, nd, bcausal};
      band.keys(myq, klo, khi);
      w_lo = band.lo(qw + 31);
      w_hi = band.hi(qw);
      const int b_hi = band.hi(min(q0 + kBR, Tq) - 1);
      ntile = min(ntile, b_hi < 0 ? 0 : b_hi / BC + 1);
      jfirst = max(0, band.lo(q0)) / BC;
    }
    // visited key blocks, as in fwd_bf16_kernel: all from jfirst on, or (block
    // mask) those whose 128-key mask block is kept for this 128-row block;
    // next_tile(j) is the first visited block at or after j (ntile when none is
    // left, or j itself past the sweep without a mask)
    const uint8_t* mrow = MASKED ? bmask + (bh % H) * mask_hstride + (long long)qb * nmk : nullptr;
    const int nvw = (nmk + 63) >> 6;
    int cw = -1;
    unsigned long long cbits = 0;
    auto word = [&](int w) {
      if (w != cw) {
        cw = w;
        cbits = mask_word(mrow, 1, nmk, w, lane);
      }
      return cbits;
    };
    auto next_tile = [&](int j) {
      if constexpr (MASKED) {
        if (j >= ntile) return ntile;
        const int c = (j * BC) >> 7;
        int w = c >> 6;
        unsigned long long bits = word(w) & (~0ull << (c & 63));
        while (bits == 0) {
          if (++w >= nvw) return ntile;
          bits = word(w);
        }
        const int c2 = w * 64 + (int)__builtin_ctzll(bits);
        return c2 == c ? j : min(ntile, (c2 << 7) / BC);
      } else {
        return j;
      }
    };
    // causal: key blocks wholly past the slice's rows add exact zeros, and both
    // waves of the slice skip them
    auto slice_sees = [&](int j) { return !CAUSAL || j * BC <= qw + 31; };
    const int j0 = next_tile(jfirst);
    char* const fslot0 = smem + L::F_OFF + ws * L::F_WAVE;   // slot s: + s * F_SLOT

    if (wave < 4) {
      // ============================ score waves ============================
      const rsrc_t rq = make_rsrc(Q + qbase, (unsigned)Tq * D * 2u);
      bf16x8 qf[L::NDS];
#pragma unroll
      for (int ds = 0; ds < L::NDS; ++ds)
        qf[ds] = as_bf16x8(bload16(rq, ((unsigned)myq * D + ds * 16 + 8 * hf) * 2u));
      const int kswz_l = kswz<L::NC>(lq);
      const int kbase_lane = lq * D * 2 + (((kswz_l >> 1) << 5) | ((hf ^ (kswz_l & 1)) << 4));
      float m_ref = -INFINITY, l_part = 0.f, lr_part = 0.f;
      barrier_keep_vmem();
      // step k of the sweep: key block j, in stage k % 4, fragments into slot k % 2
      for (int j = j0, k = 0; j < ntile; j = next_tile(j + 1), ++k) {
        if (slice_sees(j)) {
          const char* kst = stage_ptr(k & (L::NSTAGE - 1)) + L::K_OFF;
          f32x16 s;
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
          for (int ds = 0; ds < L::NDS; ++ds) s = mfma32(as_bf16x8(ld16(kst + (kbase_lane ^ (ds << 5)))), qf[ds], s);
          sched_reads_ahead<L::NDS>();
          const int k0 = j * BC;
          if constexpr (BAND != 0) {
            // outside the band of some row of the slice (or the key tail): element mask
            if (!(k0 >= w_lo && k0 + BC - 1 <= w_hi && k0 + BC <= Tk)) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = k0 + 8 * (r >> 2) + 4 * hf + (r & 3);
                if (key >= Tk || key < klo || key > khi) s[r] = -INFINITY;
              }
            }
          } else if ((CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > Tk)) {
            int lim = Tk - 1 - k0;
            if (CAUSAL) lim = min(lim, myq - k0);
            lim -= 4 * hf;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const unsigned m = (unsigned)((lim - (8 * (r >> 2) + (r & 3))) >> 31);
              const float x = s[r];
              s[r] = __builtin_bit_cast(float, (m & 0xff800000u) | (~m & __builtin_bit_cast(unsigned, x)));
            }
          }
          bf16x8 pf[2];
          float ps[4], prs[4];
          auto weights = [&](float mneg) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ps[e] = -0.f;
              prs[e] = 0.f;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              u32x4 w;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 8 * t + 2 * e;
                const float p0 = fast_exp2(__builtin_fmaf(s[r], cl2e, mneg));
                const float p1 = fast_exp2(__builtin_fmaf(s[r + 1], cl2e, mneg));
                ps[e] += p0 + p1;
                w[e] = pack_bf16(p0, p1);
                prs[e] = add_bf16_pair(w[e], prs[e]);
              }
              pf[t] = as_bf16x8(w);
            }
          };
          char* fb = fslot0 + (k & 1) * L::F_SLOT;
          bool rescale = false;
          float alpha = 1.f;
          bool need_max = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0ull;
          if (!need_max) {
            weights(-m_ref);
            const float share = (ps[0] + ps[1]) + (ps[2] + ps[3]);
            need_max = __builtin_amdgcn_ballot_w64(!(share <= kMaxWeight)) != 0ull;
          }
          if (need_max) {
            float mq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) mq[q] = max2f(max3f(s[4 * q], s[4 * q + 1], s[4 * q + 2]), s[4 * q + 3]);
            float mx = max2f(max3f(mq[0], mq[1], mq[2]), mq[3]);
            mx = half_swap_max(mx) * cl2e;
            const bool grow = mx > m_ref + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
              alpha = grow ? fast_exp2(m_ref - mx) : 1.f;
              if (grow) m_ref = mx;
              l_part *= alpha;
              lr_part *= alpha;
              rescale = true;
            }
            weights((m_ref == -INFINITY) ? 0.f : -m_ref);
          }
          l_part += (ps[0] + ps[1]) + (ps[2] + ps[3]);
          lr_part += (prs[0] + prs[1]) + (prs[2] + prs[3]);
          st16(fb + lane * 16, __builtin_bit_cast(u32x4, pf[0]));
          st16(fb + 1024 + lane * 16, __builtin_bit_cast(u32x4, pf[1]));
          reinterpret_cast<float*>(fb + 2048)[lane] = alpha;
          if (lane == 0) reinterpret_cast<unsigned*>(fb + 2304)[0] = rescale ? 1u : 0u;
        }
        wait_lds_all();
        barrier_keep_vmem();
      }
      // lse, and 1/l~ for the PV wave
      const float l_tot = half_swap_sum(l_part);
      const float lr_tot = half_swap_sum(lr_part);
      // a row that sees no key (possible only under a block mask or a band) gets O = 0, lse = -inf
      constexpr bool EMPTY_ROWS = MASKED || BAND != 0;
      reinterpret_cast<float*>(smem + L::E_OFF + ws * 256)[lane] = (!EMPTY_ROWS || lr_tot > 0.f) ? 1.f / lr_tot : 0.f;
      if (hf == 0 && myq < Tq)
        lse[(size_t)bh * Tq + myq] = (!EMPTY_ROWS || l_tot > 0.f) ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
      wait_lds_all();
      barrier_keep_vmem();
    } else {
      // ============================== PV waves =============================
      // Copies: waves 4-5 move K_j, waves 6-7 V_j (lane l of copy g moves chunk
      // 64 g + l: row s / NC, stored chunk s % NC, which holds source chunk
      // (s % NC) ^ swizzle(row), the K and V swizzles of fwd_bf16_kernel).
      const int gw = wave - 4;
      const bool is_v = gw >= 2;
      const uint16_t* const src = is_v ? V : K;
      unsigned coff[L::COPIES];
#pragma unroll
      for (int i = 0; i < L::COPIES; ++i) {
        const int sidx = ((gw & 1) * L::COPIES + i) * 64 + lane;
        const int row = sidx / L::NC, cp = sidx % L::NC;
        coff[i] = (unsigned)(row * D + (cp ^ (is_v ? vswz<L::NC>(row) : kswz<L::NC>(row))) * 8) * 2u;
      }
      const unsigned* const co = coff;   // (the host compiler drops a kernel whose lambdas index a captured array)
      const unsigned lds0 = (unsigned)(size_t)smem;
      const unsigned c_dst = (is_v ? L::V_OFF : L::K_OFF) + (gw & 1) * L::COPIES * 1024;
      auto copy_tile = [&](int j, int st) {
        const int k0 = j < ntile ? j * BC : Tk;
        const int rows = Tk - k0;
        const u32x4 r = raw_rsrc(src + kbase + (size_t)(k0 < Tk ? k0 : 0) * D, rows > 0 ? (unsigned)rows * D * 2u : 0u);
        const unsigned base = lds0 + (unsigned)st * L::STAGE + c_dst;
#pragma unroll
        for (int i = 0; i < L::COPIES; ++i) dma16_unseen(r, co[i], base + i * 1024);
      };
      const int vg = lane >> 4, vi = lane & 15;
      const int vrow = 4 * (vg >> 1) + (vi >> 2);
      const int vc0 = 2 * (vg & 1) + ((vi & 3) >> 1);
      const int vlane = vrow * L::RB + ((vc0 ^ vswz<L::NC>(vrow)) << 4) + 8 * (vi & 1);
      f32x16 o[L::NDB];
#pragma unroll
      for (int db = 0; db < L::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
      // O~^T += V_j^T P~_j^T for the block in stage st with its fragments in slot fs
      auto pv_step = [&](int st, int fs) {
        const char* fb = fslot0 + fs * L::F_SLOT;
        if (reinterpret_cast<const unsigned*>(fb + 2304)[0] != 0u) {
          const float alpha = reinterpret_cast<const float*>(fb + 2048)[lane];
#pragma unroll
          for (int db = 0; db < L::NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
        const bf16x8 p0 = as_bf16x8(ld16(fb + lane * 16)), p1 = as_bf16x8(ld16(fb + 1024 + lane * 16));
        const char* vs = stage_ptr(st) + L::V_OFF;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < L::NDB; ++db) {
            const char* p = vs + (16 * t) * L::RB + (vlane ^ (db << 6));
            const u32x2 lo = ld8_tr(p), hi = ld8_tr(p + 8 * L::RB);
            o[db] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), t ? p1 : p0, o[db]);
          }
        sched_read_pairs_ahead<2 * L::NDB, 4, 2>();
      };
      // the blocks of steps 1 and 2 (copied next), and of the previous step
      int j1 = next_tile(j0 + 1);
      int j2 = next_tile(j1 + 1);
      copy_tile(j0, 0);
      copy_tile(j1, 1);
      wait_vmem_le<L::COPIES>();
      barrier_keep_vmem();
      int jprev = -1, kprev = -1;
      for (int j = j0, k = 0; j < ntile; j = next_tile(j + 1), ++k) {
        copy_tile(j2, (k + 2) & (L::NSTAGE - 1));
        j2 = next_tile(j2 + 1);
        if (jprev >= 0 && slice_sees(jprev)) pv_step(kprev & (L::NSTAGE - 1), kprev & 1);
        jprev = j;
        kprev = k;
        wait_vmem_le<L::COPIES>();
        wait_lds_all();
        barrier_keep_vmem();
      }
      if (jprev >= 0 && slice_sees(jprev)) pv_step(kprev & (L::NSTAGE - 1), kprev & 1);
      wait_vmem_all();                                 // no copy may land after the block is done
      wait_lds_all();
      barrier_keep_vmem();                             // the score wave's 1/l~ is in LDS
      if (qw >= Tq || myq >= Tq) continue;
      const float inv = reinterpret_cast<const float*>(smem + L::E_OFF + ws * 256)[lane];
#pragma unroll
      for (int db = 0; db < L::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * hf;
          const size_t off = qbase + (size_t)myq * D + d0;
          if (OUT_F32) {
            const f32x4 w = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(static_cast<float*>(O) + off) = w;
          } else {
            u32x2 w;
            w[0] = pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
            w[1] = pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
            st8(static_cast<uint16_t*>(O) + off, w);
          }
        }
    }
  }
}

template <int D, bool CAUSAL, bool OUT_F32, bool MASKED, int BAND>
void launch_one(dim3 grid, hipStream_t stream, const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                float* lse, int Tq, int Tk, float cl2e, int nqb, const uint8_t* bmask, int H, long long hstride,
                int nmk, int wl = 0, int wr = 0, const int* cu = nullptr, int nd = 0, int bcausal = 0) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, OUT_F32, MASKED, BAND>), grid, dim3(256), 0, stream, q, k, v, o, lse,
                     Tq, Tk, cl2e, nqb, bmask, H, hstride, nmk, wl, wr, cu, nd, bcausal);
}

template <int D, bool MASKED>
void launch_dtype(dim3 grid, hipStream_t stream, int causal, int out_f32, const uint16_t* q, const uint16_t* k,
                  const uint16_t* v, void* O, float* lse, int Tq, int Tk, float cl2e, int nqb, const uint8_t* bmask,
                  int H, long long hstride, int nmk) {
  if (causal) {
    if (out_f32) launch_one<D, true, true, MASKED, 0>(grid, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, bmask, H, hstride, nmk);
    else launch_one<D, true, false, MASKED, 0>(grid, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, bmask, H, hstride, nmk);
  } else {
    if (out_f32) launch_one<D, false, true, MASKED, 0>(grid, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, bmask, H, hstride, nmk);
    else launch_one<D, false, false, MASKED, 0>(grid, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, bmask, H, hstride, nmk);
  }
}

template <int D>
int launch(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H, int Tq, int Tk,
           float scale, int causal, int out_f32, const uint8_t* bmask, int mask_heads, int band, int wl, int wr,
           const int* cu, int nd, hipStream_t stream) {
  const int nqb = (Tq + kBR - 1) / kBR;
  const long long nblk = (long long)nqb * B * H;
  if (nblk > 0x7fffffffLL) return FA_ERR_SHAPE;
  const float cl2e = scale * kLog2e;
  const dim3 grid((unsigned)nblk);
  auto q = static_cast<const uint16_t*>(Q);
  auto k = static_cast<const uint16_t*>(K);
  auto v = static_cast<const uint16_t*>(V);
  // block mask [mask_heads][ceil(Tq/128)][ceil(Tk/128)]; the 128-row blocks are this kernel's query blocks
  const int nmk = (Tk + 127) / 128;
  const long long hstride = mask_heads == 1 ? 0 : (long long)nqb * nmk;
  // plain causal: query blocks nqb-1-p and p share a workgroup
  const dim3 pgrid((unsigned)((long long)((nqb + 1) / 2) * B * H));
  if constexpr (D == 256) {
    // every mask form in two roles, eight waves per 128-row block
    auto go = [&](auto kernel, dim3 g) {
      hipLaunchKernelGGL(kernel, g, dim3(512), 0, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, bmask, H, hstride, nmk,
                         wl, wr, cu, nd, causal);
    };
    if (band == 1) {
      if (out_f32) go(fwd_split_kernel<D, false, true, false, 1>, grid);
      else go(fwd_split_kernel<D, false, false, false, 1>, grid);
    } else if (band == 2) {
      if (out_f32) go(fwd_split_kernel<D, false, true, false, 2>, grid);
      else go(fwd_split_kernel<D, false, false, false, 2>, grid);
    } else if (bmask) {
      if (causal) {
        if (out_f32) go(fwd_split_kernel<D, true, true, true, 0>, grid);
        else go(fwd_split_kernel<D, true, false, true, 0>, grid);
      } else {
        if (out_f32) go(fwd_split_kernel<D, false, true, true, 0>, grid);
        else go(fwd_split_kernel<D, false, false, true, 0>, grid);
      }
    } else if (causal) {
      if (out_f32) go(fwd_split_kernel<D, true, true, false, 0>, pgrid);
      else go(fwd_split_kernel<D, true, false, false, 0>, pgrid);
    } else {
      if (out_f32) go(fwd_split_kernel<D, false, true, false, 0>, grid);
      else go(fwd_split_kernel<D, false, false, false, 0>, grid);
    }
  } else {
    if (band == 1) {
      if (out_f32)
        launch_one<D, false, true, false, 1>(grid, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, nullptr, H, 0, nmk, wl, wr);
      else
        launch_one<D, false, false, false, 1>(grid, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, nullptr, H, 0, nmk, wl, wr);
    } else if (band == 2) {
      if (out_f32)
        launch_one<D, false, true, false, 2>(grid, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, nullptr, H, 0, nmk, 0, 0,
                                             cu, nd, causal);
      else
        launch_one<D, false, false, false, 2>(grid, stream, q, k, v, O, lse, Tq, Tk, cl2e, nqb, nullptr, H, 0, nmk, 0, 0,
                                              cu, nd, causal);
    } else if (bmask) {
      launch_dtype<D, true>(grid, stream, causal, out_f32, q, k, v, O, lse, Tq, Tk, cl2e, nqb, bmask, H, hstride, nmk);
    } else {
      launch_dtype<D, false>(causal ? pgrid : grid, stream, causal, out_f32, q, k, v, O, lse, Tq, Tk, cl2e, nqb,
                             nullptr, H, 0, nmk);
    }
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int launch_fwd_bf16(const void* Q, const void* K, const void* V, void* O, float* lse, int B, int H,
                    int Tq, int Tk, int d, float scale, int causal, int out_f32, hipStream_t stream,
                    const uint8_t* bmask, int mask_heads, int band, int wl, int wr, const int* cu, int nd) {
  switch (d) {
    case 64: return launch<64>(Q, K, V, O, lse, B, H, Tq, Tk, scale, causal, out_f32, bmask, mask_heads, band, wl, wr, cu, nd, stream);
    case 128: return launch<128>(Q, K, V, O, lse, B, H, Tq, Tk, scale, causal, out_f32, bmask, mask_heads, band, wl, wr, cu, nd, stream);
    case 256: return launch<256>(Q, K, V, O, lse, B, H, Tq, Tk, scale, causal, out_f32, bmask, mask_heads, band, wl, wr, cu, nd, stream);
    default: return FA_ERR_HEADDIM;
  }
}

}  // namespace fa
