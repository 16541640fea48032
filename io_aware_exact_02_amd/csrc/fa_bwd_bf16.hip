// Backward pass for bf16 inputs on gfx950 MFMA.
//
// [ZtF] = "FlashAttention", zerotofrontier.app textbook section 12.3,
// sections "The backward pass, derived" and "Which loop goes outside?".
//
// Every kernel here starts from the row terms D = rowsum(dO * O) that a
// pre-pass leaves in the workspace (Observation 2) and rebuilds the weights
// from lse as P = exp2(S * scale*log2e - lse*log2e) (Observation 1).
//
// Every head width: two sweeps, no atomics, each output summed in a fixed
// order ([ZtF] "Which loop goes outside?"):
//   * key-block sweep: one workgroup per block of 128 keys sweeps the query
//     tiles and writes dK_j and dV_j once (bwd_kv_kernel for d = 64 and 128,
//     bwd_kv_w4_kernel for d = 256);
//   * query-block sweep (bwd_dq_kernel): one workgroup per block of queries
//     sweeps the key blocks and writes dQ_i once.
// Under a plain causal mask a workgroup runs two blocks in turn, a short sweep
// and a long one, so that all workgroups are about equally long (the key-block
// sweep does so at d = 128); workgroups of unequal length leave CUs idle,
// waiting on the dispatcher.
// The split forms S and dP twice (seven tile products instead of five) but
// sends no dQ traffic beyond one write: adding each key block's share of dQ
// with float32 atomics would send Tk/128 partial sums per dQ element through
// the memory-side atomic units, which is slower on this part than recomputing.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kKeysPerWave = 32;
constexpr int kWavesB = 4;
constexpr int kBKC = kKeysPerWave * kWavesB;   // keys per workgroup
constexpr int kBQ = 32;                        // query rows per step

// Block-sparse sweeps ([ZtF] "Dropout, block-sparsity, and other real-kernel
// details"): the mask holds one byte per (128-query block, 128-key block).  A
// key block's workgroup visits only the query tiles whose block keeps it; each
// wave reads its mask column 64 blocks at a time as a bit word (a ballot, held
// in scalar registers) and walks the visible tiles with its own cursor.  Every
// wave derives the same sequence, so all waves pass the same number of
// barriers.
constexpr int kMaskBlock = 128;
constexpr int kTilesPerMaskRow = kMaskBlock / kBQ;
static_assert(kBKC == kMaskBlock, "one key-block workgroup per mask column");

// The query tiles a key-block sweep visits, shared by both key-block kernels:
// all tiles from it0 on, those before nqe (band masks), or (block masks) those
// whose 128-query block keeps this key block.  count() is their number, next(t)
// the first visible tile >= t (nqt when none is left).  Every lane of the wave
// must be active in both.
template <bool MASKED, bool BANDED = false>
struct KeyBlockTiles {
  const uint8_t* mcol;     // mask column of this key block (stride nmk), MASKED only
  int nmk, nmq, nvw, nqt, it0, lane;
  int nqe = 0;             // BANDED: one past the last query tile that sees the block
  int cw = -1;             // the word last read is kept in scalar registers
  unsigned long long cbits = 0;

  __device__ KeyBlockTiles(const uint8_t* bmask, long long head_off, int kblk, int nmk_, int Tq, int it0_, int lane_)
      : mcol(MASKED ? bmask + head_off + kblk : nullptr), nmk(nmk_), nmq((Tq + kMaskBlock - 1) / kMaskBlock),
        nvw((nmq + 63) >> 6), nqt((Tq + kBQ - 1) / kBQ), it0(it0_), lane(lane_) {}
  // bit r of word w: query block 64w + r keeps this key block
  __device__ unsigned long long word(int w) {
    if (w != cw) {
      cw = w;
      cbits = mask_word(mcol, nmk, nmq, w, lane);
    }
    return cbits;
  }
  __device__ bool row(int r) { return ((word(r >> 6) >> (r & 63)) & 1ull) != 0; }
  __device__ int next_row(int r) {               // first visible query block >= r, nmq if none
    int w = r >> 6;
    if (w >= nvw) return nmq;
    unsigned long long bits = word(w) & (~0ull << (r & 63));
    while (bits == 0) {
      if (++w >= nvw) return nmq;
      bits = word(w);
    }
    return w * 64 + (int)__builtin_ctzll(bits);
  }
  __device__ int next(int t) {
    if constexpr (BANDED) return t < nqe ? t : nqt;
    if constexpr (MASKED) {
      if (t >= nqt) return nqt;
      if (row(t / kTilesPerMaskRow)) return t;
      const int r = next_row(t / kTilesPerMaskRow + 1);
      return r < nmq ? r * kTilesPerMaskRow : nqt;
    } else {
      return t;
    }
  }
  __device__ int count() {
    if constexpr (MASKED) {
      if (it0 >= nqt) return 0;
      const int rlo = it0 / kTilesPerMaskRow;
      int n = 0;
      for (int w = rlo >> 6; w < nvw; ++w) {
        unsigned long long bits = word(w);
        if (w == (rlo >> 6)) bits &= ~0ull << (rlo & 63);
        n += __builtin_popcountll(bits);
      }
      n *= kTilesPerMaskRow;
      if (row(rlo)) n -= it0 - rlo * kTilesPerMaskRow;           // the first block starts at it0
      if (row(nmq - 1)) n -= nmq * kTilesPerMaskRow - nqt;       // the last block is ragged
      return n;
    } else if constexpr (BANDED) {
      return max(0, nqe - it0);
    } else {
      return nqt - it0;
    }
  }
};

// ---------------------------------------------------------------------------
// Chunk swizzle of row r of a row-major bf16 tile held in LDS (16-byte chunk c
// of row r is stored at chunk c ^ row_swz(r)), for two kinds of reads.  Row
// reads (16 lanes = 16 consecutive rows, one 16-byte chunk each) need the
// swizzle to be a permutation over any 16 rows (for 128-byte rows, two per
// 256-byte bank cycle: over the row pairs).  Transposing reads (a half-wave = 4
// consecutive rows x 4 chunks, 8 bytes per lane) need the four rows to spread
// a chunk group over all bank groups: the row's position among the four moves
// chunk bits 2-3 (for 128-byte rows, the odd row pair flips bit 2).  The
// swizzle changes chunk bits >= 2 only through the row, so a 32-feature
// block's offset is a XOR with (db << 6).
// ---------------------------------------------------------------------------
template <int NC>
__device__ __forceinline__ int row_swz(int r) {
  if constexpr (NC == 8) {
    const int u = (r >> 1) & 7;
    return u ^ ((u & 1) << 2);
  } else {
    return 4 * (r & 3) + ((r >> 2) & 3);
  }
}

// ---------------------------------------------------------------------------
// Key-block sweep for d = 256 (bwd_kv_w4_kernel): dK_j and dV_j.
//
// Four waves, one per SIMD, each owning 32 keys: K_j, V_j (MFMA B operands)
// and the float32 accumulators dK_j, dV_j stay in registers (the accumulators
// alone take 256 per lane, so two waves per SIMD do not fit).  Per query tile
// i of 32 rows, in a ring of three LDS stages:
//   * Q_i, dO_i, Ln_i and Dn_i (the negated row terms) go HBM -> LDS by
//     buffer_load ... lds two tiles ahead, Q_i and dO_i rows chunk-swizzled
//     (row_swz).  One row-major copy serves both kinds of product: row reads
//     for those over features, transposing 8-byte reads (one feature per lane,
//     queries in the k-slot order of the P and dS fragments) for those over
//     queries.
//   * S = Q_i K_j^T and dP = dO_i V_j^T with one key per lane; P = exp2(S c
//     log2e + Ln_i) and dS = P (dP + Dn_i) ([ZtF] "The backward pass,
//     derived", Observations 1-3); only tiles crossing the causal diagonal
//     are masked.  Rows past Tq and keys past Tk read as zeros and add nothing.
//   * dV_j += P^T dO_i and dK_j += dS^T Q_i with P and dS straight from
//     registers.
// The copies are issued in inline assembly, out of the compiler's sight: it
// cannot tell the stages of one LDS array apart and would otherwise wait for
// every copy in flight before each transposing read.  The kernel does its own
// waiting: before the barrier that closes a step, each wave waits for its
// copies of the next tile (the copies complete in issue order).
// dQ comes from the query-block sweep below, as for the narrower heads.
// ---------------------------------------------------------------------------
template <int D>
struct W4Layout {
  static constexpr int NC = D / 8;              // 16-byte chunks per row
  static constexpr int RB = D * 2;              // bytes per row
  static constexpr int TB = kBQ * RB;           // one Q or dO tile
  static constexpr int Q_OFF = 0;               // byte offsets inside one stage
  static constexpr int G_OFF = TB;
  static constexpr int L_OFF = 2 * TB;          // Ln: 64 floats (the second 32 unused)
  static constexpr int D_OFF = L_OFF + 256;     // Dn: likewise
  static constexpr int X_OFF = D_OFF + 256;     // waves 2 and 3 copy their row terms here, unused
  static constexpr int STAGE = X_OFF + 512;
  static constexpr int NSTAGE = 3;
  static constexpr int BYTES = NSTAGE * STAGE;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int DMA_W = TB / 1024 / 2;   // 1 KiB copies per wave and tensor (two waves per tensor)
  static constexpr int COPIES = DMA_W + 1;      // copies a wave issues per tile
  static_assert(NC >= 16, "row_swz of 16 or more chunks");
  static_assert(STAGE % 1024 == 0 && COPIES <= 15, "stage alignment; vmcnt field");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int D, bool CAUSAL, bool MASKED, int BAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_kv_w4_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                      const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                      const float* __restrict__ Ln, const float* __restrict__ Dn,
                      void* __restrict__ dK, void* __restrict__ dV, int Tq, int Tk, float scale, float cl2e,
                      int nkb, int grad_f32, const uint8_t* __restrict__ bmask, int H, long long mask_hstride,
                      int nmk, int wl, int wr, const int* __restrict__ cu, int nd, int bcausal) {
  using L = W4Layout<D>;
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];

  const int nblk = gridDim.x, wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int bh = lin / nkb;
  const int kblk = lin % nkb;   // causal: key block 0 has the longest sweep, so it goes first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  const int k0 = kblk * kBKC;
  const int kw0 = k0 + wave * kKeysPerWave;
  const int mykey = kw0 + l32;

  const rsrc_t rk = make_rsrc(K + kbase, (unsigned)Tk * D * 2u);
  const rsrc_t rv = make_rsrc(V + kbase, (unsigned)Tk * D * 2u);

  // K_j and V_j as B operands (column = key, k = features), held for the sweep.
  bf16x8 kf[L::NDS], vf[L::NDS];
#pragma unroll
  for (int ds = 0; ds < L::NDS; ++ds) {
    const unsigned off = ((unsigned)mykey * D + ds * 16 + 8 * hf) * 2u;
    kf[ds] = as_bf16x8(bload16(rk, off));
    vf[ds] = as_bf16x8(bload16(rv, off));
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
  // BAND: the queries that see this block's keys, and those that see every key
  // of this wave (a tile between them needs no element mask), from the key side
  const Band<BAND> band{wl, wr, cu, nd, bcausal};
  int w_qlo = 0, w_qhi = 0, my_qlo = 0, my_qhi = 0;   // and this lane's key: my_qlo .. my_qhi
  if constexpr (BAND != 0) {
    w_qlo = band.qlo(kw0 + kKeysPerWave - 1);
    w_qhi = band.qhi(kw0);
    band.queries(mykey, my_qlo, my_qhi);
  }
  const int it0 = BAND != 0 ? min(max(0, band.qlo(k0)) / kBQ, nqt) : CAUSAL ? min(k0 / kBQ, nqt) : 0;
  KeyBlockTiles<MASKED, BAND != 0> tiles(bmask, (long long)(bh % H) * mask_hstride, kblk, nmk, Tq, it0, lane);
  if constexpr (BAND != 0) {
    const int qh = band.qhi(min(k0 + kBKC, Tk) - 1);
    tiles.nqe = qh < 0 ? 0 : min(nqt, qh / kBQ + 1);
  }
  const int n = tiles.count();                  // query tiles in the sweep

  // ---- copies of one query tile into a stage.  Waves 0-1 move Q_i, waves 2-3
  // dO_i: lane l of copy g (0 .. 2 DMA_W - 1 over the tensor's two waves) moves
  // chunk s = 64 g + l of the tile, row s / NC, stored at chunk s % NC, which
  // holds source chunk (s % NC) ^ row_swz(row).  Wave 0 also copies Ln_i and
  // wave 1 Dn_i (64 floats from the tile's first row); waves 2 and 3 make the
  // same copies into an unused slot, so that every wave issues COPIES per tile.
  // The lane offsets do not change between tiles; the tile's first row goes
  // into a buffer resource over rows r0 .. Tq-1, so rows past Tq -- and whole
  // tiles past the sweep, which start at row Tq -- read as zeros.
  const bool is_g = wave >= 2;
  const uint16_t* const src = is_g ? dO : Q;
  unsigned coff[L::DMA_W];
#pragma unroll
  for (int i = 0; i < L::DMA_W; ++i) {
    const int s = ((wave & 1) * L::DMA_W + i) * 64 + lane;
    const int row = s / L::NC, cp = s % L::NC;
    coff[i] = (unsigned)(row * D + (cp ^ row_swz<L::NC>(row)) * 8) * 2u;
  }
  const unsigned* const co = coff;   // (the host compiler drops a kernel whose lambdas index a captured array)
  const float* const terms = ((wave & 1) ? Dn : Ln) + (size_t)bh * Tq;
  const unsigned lds0 = (unsigned)(size_t)smem;
  const unsigned t_dst = (wave & 1) ? L::D_OFF : L::L_OFF;
  const unsigned x_dst = is_g ? L::X_OFF + 256 * (wave & 1) : t_dst;
  const unsigned c_dst = (is_g ? L::G_OFF : L::Q_OFF) + (wave & 1) * L::DMA_W * 1024;
  auto tile_row = [&](int t) { return t < nqt ? t * kBQ : Tq; };
  auto copy_tile = [&](int t, int st) {
    const int r0 = tile_row(t);
    const int rows = Tq - r0;
    const unsigned base = lds0 + (unsigned)st * L::STAGE;
    const u32x4 r = raw_rsrc(src + qbase + (size_t)(r0 < Tq ? r0 : 0) * D, rows > 0 ? (unsigned)rows * D * 2u : 0u);
#pragma unroll
    for (int i = 0; i < L::DMA_W; ++i) dma16_unseen(r, co[i], base + c_dst + i * 1024);
    const u32x4 rt = raw_rsrc(terms + (r0 < Tq ? r0 : 0), rows > 0 ? (unsigned)rows * 4u : 0u);
    dma4_unseen(rt, (unsigned)lane * 4u, base + x_dst);
  };

  // this lane's row read for k-step ds: chunk (2 ds + hf) ^ swz of row l32
  const int swz_l = row_swz<L::NC>(l32);
  const int n_lane = l32 * L::RB + (((swz_l >> 1) << 5) | ((hf ^ (swz_l & 1)) << 4));
  // transposing reads (B operands of the products over queries): lane l gets
  // feature 32 db + l % 32, queries 16 t + 4 hf + 0..3 and 16 t + 8 + 4 hf +
  // 0..3 of the tile -- the k-slot order of the P and dS fragments.  Each half
  // comes from one read in which lane 16 g + 4 e + j addresses query row
  // 4 (g / 2) + e (+ 8 for the second half) and features 16 (g % 2) + 4 j ..
  // +3; tb[sec] is that offset for t = db = 0.
  const int tg = lane >> 4, ti = lane & 15;
  int tb[2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int row = 8 * sec + 4 * (tg >> 1) + (ti >> 2);
    const int c = 2 * (tg & 1) + ((ti & 3) >> 1);
    tb[sec] = row * L::RB + ((c ^ row_swz<L::NC>(row)) << 4) + 8 * (ti & 1);
  }
  auto tr_operand = [&](const char* tile, int t, int db) {
    const char* base = tile + t * 16 * L::RB;
    const u32x2 lo = ld8_tr(base + (tb[0] ^ (db << 6)));
    const u32x2 hi = ld8_tr(base + (tb[1] ^ (db << 6)));
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  };

  // tile t in stage st; tile tf is copied into stage sf (two steps ahead)
  auto step = [&](int t, int st, int tf, int sf) {
    copy_tile(tf, sf);
    const int r0 = t * kBQ;
    const char* sb_ = smem + st * L::STAGE;

    // S = Q_i K_j^T and dP = dO_i V_j^T: lane = key, register r = query 8(r/4)+4hf+r%4
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int ds = 0; ds < L::NDS; ++ds) {
      const int off = n_lane ^ (ds << 5);
      const bf16x8 a = as_bf16x8(ld16(sb_ + L::Q_OFF + off));
      s = mfma32(a, kf[ds], s);
      const bf16x8 g = as_bf16x8(ld16(sb_ + L::G_OFF + off));
      dp = mfma32(g, vf[ds], dp);
    }
    sched_reads_ahead<2 * L::NDS>();
    const float* lsv = reinterpret_cast<const float*>(sb_ + L::L_OFF);
    const float* dsv_ = reinterpret_cast<const float*>(sb_ + L::D_OFF);
    float p[16], dsv[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int qr = 8 * g4 + 4 * hf;
      const f32x4 lv = *reinterpret_cast<const f32x4*>(lsv + qr);
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(dsv_ + qr);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g4 + e;
        p[r] = fast_exp2(__builtin_fmaf(s[r], cl2e, lv[e]));
        dsv[r] = dp[r] + dv4[e];
      }
    }
    if (CAUSAL && r0 < kw0 + kKeysPerWave - 1) {       // the tile crosses this wave's diagonal
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (mykey > r0 + 8 * (r >> 2) + 4 * hf + (r & 3)) p[r] = 0.f;
    }
    if (BAND != 0 && !(r0 >= w_qlo && r0 + kBQ - 1 <= w_qhi)) {   // crosses a band edge
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = r0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (qr < my_qlo || qr > my_qhi) p[r] = 0.f;
      }
    }
    bf16x8 pb[2], sbf[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      u32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * t2 + 2 * e;
        a[e] = pack_bf16(p[r], p[r + 1]);
        b[e] = pack_bf16(p[r] * dsv[r], p[r + 1] * dsv[r + 1]);
      }
      pb[t2] = as_bf16x8(a);
      sbf[t2] = as_bf16x8(b);
    }
    // dV_j += P^T dO_i ; dK_j += dS^T Q_i  (lane = feature column, register = key row)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int db = 0; db < L::NDB; ++db) {
        dv[db] = mfma32(pb[t2], tr_operand(sb_ + L::G_OFF, t2, db), dv[db]);
        dk[db] = mfma32(sbf[t2], tr_operand(sb_ + L::Q_OFF, t2, db), dk[db]);
      }
    sched_read_pairs_ahead<4 * L::NDB>();
    // the next tile's copies (issued a step ago) have landed, for every wave;
    // this step's reads are done before any wave copies over this stage
    wait_vmem_le<L::COPIES>();
    wait_lds_all();
    barrier_keep_vmem();
  };

  int t0 = tiles.next(it0);                     // tiles of the next two steps
  int t1 = tiles.next(t0 + 1);
  copy_tile(t0, 0);
  copy_tile(t1, 1);
  wait_vmem_le<L::COPIES>();
  barrier_keep_vmem();
  for (int s = 0, st = 0; s < n; ++s) {
    const int t2 = tiles.next(t1 + 1);
    const int sf = st == 0 ? 2 : st - 1;        // (st + 2) % 3
    step(t0, st, t2, sf);
    t0 = t1;
    t1 = t2;
    st = st == 2 ? 0 : st + 1;
  }
  wait_vmem_all();                              // no copy may land after the workgroup has left

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
//     lane).
//   * gradient waves 4-7 (wave 4+w serves score wave w's keys) keep dV_j and
//     dK_j in float32 registers and trail the score waves by one query tile:
//     dV_j += P^T dO_i and dK_j += dS^T Q_i.  They also issue the copies.
// Q_i, dO_i, Ln_i and Dn_i (the negated row terms) go HBM -> LDS by
// buffer_load ... lds, two tiles ahead, into a ring of four stages (the score
// waves read tile i's while the gradient waves read tile i-1's, tile i+1's has
// landed and tile i+2's is in flight); Q_i and dO_i rows are chunk-swizzled
// (row_swz).  One row-major copy serves both roles: row reads for the score
// waves' products over features, transposing 8-byte reads (one feature per
// lane, queries in the k-slot order of the fragments) for the gradient waves'
// products over queries.  The copies are issued in inline assembly, which the
// compiler does not see, so it adds no wait for them before LDS reads of other
// stages; the gradient waves wait for their own copies of the next tile before
// the barrier that closes a phase.  One bare s_barrier per phase orders
// everything, after the wave's own LDS writes (the fragments) have completed.
// Rows past Tq and keys past Tk need no masking: their Q/dO or K/V rows read
// as zeros, so they add nothing to the gradients that are stored.
// ---------------------------------------------------------------------------
template <int D>
struct KvLayout {
  static constexpr int NC = D / 8;                           // 16-byte chunks per row
  static constexpr int RB = D * 2;                           // bytes per row
  static constexpr int TB = kBQ * RB;                        // one Q or dO tile
  static constexpr int Q_OFF = 0;                            // byte offsets inside one stage
  static constexpr int G_OFF = TB;
  static constexpr int L_OFF = 2 * TB;                       // Ln: 64 floats (the second 32 unused)
  static constexpr int D_OFF = L_OFF + 256;                  // Dn: likewise
  static constexpr int X_OFF = D_OFF + 256;                  // gradient waves 6 and 7 copy row terms here, unused
  static constexpr int STAGE = X_OFF + 512;
  static constexpr int NSTAGE = 4;
  static constexpr int F_OFF = NSTAGE * STAGE;               // fragments, two slots
  static constexpr int F_WAVE = 4 * 64 * 16;                 // P^T and dS^T fragments of one score wave
  static constexpr int F_BYTES = kWavesB * F_WAVE;
  static constexpr int BYTES = F_OFF + 2 * F_BYTES;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int DMA_W = TB / 1024 / 2;                // 1 KiB copies per gradient wave (two per tensor)
  static constexpr int COPIES = DMA_W + 1;                   // copies a gradient wave issues per tile
  static_assert(STAGE % 1024 == 0 && COPIES <= 15, "stage alignment; vmcnt field");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int D, bool CAUSAL, bool MASKED, int BAND>
__global__ __launch_bounds__(512) void bwd_kv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Ln, const float* __restrict__ Dn,
    void* __restrict__ dK, void* __restrict__ dV, int Tq, int Tk, float scale, float cl2e, int nkb, int grad_f32,
    const uint8_t* __restrict__ bmask, int H, long long mask_hstride, int nmk, int wl, int wr,
    const int* __restrict__ cu, int nd, int bcausal) {
  using L = KvLayout<D>;
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];

  // Plain causal at d = 128: workgroup p of a head runs key block p, then key
  // block nkb-1-p, so every workgroup sweeps about the same number of query
  // tiles (uneven workgroups leave CUs waiting on the dispatcher).  At d = 64
  // the loop over two blocks compiles to a slower sweep (2-5% measured) than
  // the dispatch gaps it removes.  Otherwise one block per workgroup; causal
  // key block 0 has the longest sweep and goes first.
  constexpr bool PAIRED = CAUSAL && !MASKED && BAND == 0 && D == 128;
  const int nblk = gridDim.x, wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int npb = PAIRED ? (nkb + 1) / 2 : nkb;     // workgroups per head
  const int bh = lin / npb;
  const int pidx = lin % npb;
  const int npass = (PAIRED && 2 * pidx + 1 < nkb) ? 2 : 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int wq = wave & 3;                      // key slice (score wave w and gradient wave 4+w)
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  auto stage_ptr = [&](int st) { return smem + st * L::STAGE; };
  for (int pass = 0; pass < npass; ++pass) {
    const int kblk = pass == 0 ? pidx : nkb - 1 - pidx;
    if (pass > 0) {
      // the gradient waves' last step read the previous block's LDS slots
      wait_lds_all();
      barrier_keep_vmem();
    }
    const int k0 = kblk * kBKC;
    const int kw0 = k0 + wq * kKeysPerWave;
    const int mykey = kw0 + l32;

    const int nqt = (Tq + kBQ - 1) / kBQ;
    // BAND: the queries that see this block's keys, and those that see every key
    // of this wave (a tile between them needs no element mask), from the key side
    const Band<BAND> band{wl, wr, cu, nd, bcausal};
    int w_qlo = 0, w_qhi = 0, my_qlo = 0, my_qhi = 0;   // and this lane's key: my_qlo .. my_qhi
    if constexpr (BAND != 0) {
      w_qlo = band.qlo(kw0 + kKeysPerWave - 1);
      w_qhi = band.qhi(kw0);
      band.queries(mykey, my_qlo, my_qhi);
    }
    const int it0 = BAND != 0 ? min(max(0, band.qlo(k0)) / kBQ, nqt) : CAUSAL ? min(k0 / kBQ, nqt) : 0;
    // tile t covers query rows t kBQ ..; a tile past the sweep reads row Tq (zeros)
    auto tile_row = [&](int t) { return t < nqt ? t * kBQ : Tq; };

    // visible query tiles: all from it0 on, or (masked) those whose block keeps this key block
    KeyBlockTiles<MASKED, BAND != 0> tiles(bmask, (long long)(bh % H) * mask_hstride, kblk, nmk, Tq, it0, lane);
    if constexpr (BAND != 0) {
      const int qh = band.qhi(min(k0 + kBKC, Tk) - 1);
      tiles.nqe = qh < 0 ? 0 : min(nqt, qh / kBQ + 1);
    }
    const int n = tiles.count();                  // query tiles in the sweep
    auto next_tile = [&](int t) { return tiles.next(t); };

    if (wave < 4) {
      // ============================ score waves ============================
      const rsrc_t rk = make_rsrc(K + kbase, (unsigned)Tk * D * 2u);
      const rsrc_t rv = make_rsrc(V + kbase, (unsigned)Tk * D * 2u);
      bf16x8 kf[L::NDS], vf[L::NDS];
#pragma unroll
      for (int ds = 0; ds < L::NDS; ++ds) {
        const unsigned off = ((unsigned)mykey * D + ds * 16 + 8 * hf) * 2u;
        kf[ds] = as_bf16x8(bload16(rk, off));
        vf[ds] = as_bf16x8(bload16(rv, off));
      }
      // this lane's row read for k-step ds: chunk (2 ds + hf) ^ swz of query row l32
      const int swz_l = row_swz<L::NC>(l32);
      const int n_lane = l32 * L::RB + (((swz_l >> 1) << 5) | ((hf ^ (swz_l & 1)) << 4));
      int tc = next_tile(it0);                      // the tile of the next score step
      barrier_keep_vmem();

      // tile t in stage st, fragments into slot fs
      for (int s = 0; s < n; ++s) {
        const int t = tc;
        tc = next_tile(tc + 1);
        const int r0 = t * kBQ;
        const char* sb_ = stage_ptr(s & (L::NSTAGE - 1));
        // -lse log2e and -D of the tile's queries in the accumulator order:
        // register r <-> query 8(r/4) + 4hf + r%4 (all lanes of a half alike)
        f32x16 lt, dp;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(sb_ + L::L_OFF + (8 * g4 + 4 * hf) * 4);
          const f32x4 b = *reinterpret_cast<const f32x4*>(sb_ + L::D_OFF + (8 * g4 + 4 * hf) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lt[4 * g4 + e] = a[e];
            dp[4 * g4 + e] = b[e];
          }
        }
        // S = Q_i K_j^T and dP - D = dO_i V_j^T - D_i: lane = key, register r = query 8(r/4)+4hf+r%4
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int ds = 0; ds < L::NDS; ++ds) {
          const int off = n_lane ^ (ds << 5);
          sacc = mfma32(as_bf16x8(ld16(sb_ + L::Q_OFF + off)), kf[ds], sacc);
          dp = mfma32(as_bf16x8(ld16(sb_ + L::G_OFF + off)), vf[ds], dp);
        }
        sched_reads_ahead<2 * L::NDS, 2 * L::NDS + 8, 6>();
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(sacc[r], cl2e, lt[r]));
        if (CAUSAL && r0 < kw0 + kKeysPerWave - 1) {     // the tile crosses this wave's diagonal
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (mykey > r0 + 8 * (r >> 2) + 4 * hf + (r & 3)) p[r] = 0.f;
        }
        if (BAND != 0 && !(r0 >= w_qlo && r0 + kBQ - 1 <= w_qhi)) {   // crosses a band edge
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qr = r0 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (qr < my_qlo || qr > my_qhi) p[r] = 0.f;
          }
        }
        // fragments for the gradient wave: [P^T t=0, P^T t=1, dS^T t=0, dS^T t=1], 1 KiB each
        char* fb = smem + L::F_OFF + (s & 1) * L::F_BYTES + wq * L::F_WAVE + lane * 16;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          u32x4 a, b;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * t2 + 2 * e;
            a[e] = pack_bf16(p[r], p[r + 1]);
            b[e] = pack_bf16(p[r] * dp[r], p[r + 1] * dp[r + 1]);
          }
          st16(fb + t2 * 1024, a);
          st16(fb + (2 + t2) * 1024, b);
        }
        // the fragments are complete, and so are this step's reads of the stage
        wait_lds_all();
        barrier_keep_vmem();
      }
    } else {
      // =========================== gradient waves ==========================
      // Copies of one tile into a stage.  Waves 4-5 move Q_i, waves 6-7 dO_i:
      // lane l of copy g (0 .. 2 DMA_W - 1 over the tensor's two waves) moves
      // chunk s = 64 g + l of the tile, row s / NC, stored at chunk s % NC,
      // which holds source chunk (s % NC) ^ row_swz(row).  Wave 4 also copies
      // Ln_i and wave 5 Dn_i (64 floats from the tile's first row); waves 6 and
      // 7 make the same copies into an unused slot, so that every gradient wave
      // issues COPIES per tile.  The lane offsets do not change between tiles;
      // the tile's first row goes into a buffer resource over rows r0 .. Tq-1,
      // so rows past Tq -- and whole tiles past the sweep, which start at row Tq
      // -- read as zeros.
      const int gw = wave - 4;
      const bool is_g = gw >= 2;
      const uint16_t* const src = is_g ? dO : Q;
      unsigned coff[L::DMA_W];
#pragma unroll
      for (int i = 0; i < L::DMA_W; ++i) {
        const int s = ((gw & 1) * L::DMA_W + i) * 64 + lane;
        const int row = s / L::NC, cp = s % L::NC;
        coff[i] = (unsigned)(row * D + (cp ^ row_swz<L::NC>(row)) * 8) * 2u;
      }
      const unsigned* const co = coff;   // (the host compiler drops a kernel whose lambdas index a captured array)
      const float* const terms = ((gw & 1) ? Dn : Ln) + (size_t)bh * Tq;
      const unsigned lds0 = (unsigned)(size_t)smem;
      const unsigned t_dst = (gw & 1) ? L::D_OFF : L::L_OFF;
      const unsigned x_dst = is_g ? L::X_OFF + 256 * (gw & 1) : t_dst;
      const unsigned c_dst = (is_g ? L::G_OFF : L::Q_OFF) + (gw & 1) * L::DMA_W * 1024;
      auto copy_tile = [&](int t, int st) {
        const int r0 = tile_row(t);
        const int rows = Tq - r0;
        const unsigned base = lds0 + (unsigned)st * L::STAGE;
        const u32x4 r = raw_rsrc(src + qbase + (size_t)(r0 < Tq ? r0 : 0) * D, rows > 0 ? (unsigned)rows * D * 2u : 0u);
#pragma unroll
        for (int i = 0; i < L::DMA_W; ++i) dma16_unseen(r, co[i], base + c_dst + i * 1024);
        const u32x4 rt = raw_rsrc(terms + (r0 < Tq ? r0 : 0), rows > 0 ? (unsigned)rows * 4u : 0u);
        dma4_unseen(rt, (unsigned)lane * 4u, base + x_dst);
      };

      // transposing reads (B operands of the products over queries): lane l gets
      // feature 32 db + l % 32, queries 16 t + 4 hf + 0..3 and 16 t + 8 + 4 hf +
      // 0..3 of the tile -- the k-slot order of the fragments.  Each half comes
      // from one read in which lane 16 g + 4 e + j addresses query row
      // 4 (g / 2) + e (+ 8 for the second half) and features 16 (g % 2) + 4 j ..
      // +3; tb[sec] is that offset for t = db = 0.
      const int tg = lane >> 4, ti = lane & 15;
      int tb[2];
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int row = 8 * sec + 4 * (tg >> 1) + (ti >> 2);
        const int c = 2 * (tg & 1) + ((ti & 3) >> 1);
        tb[sec] = row * L::RB + ((c ^ row_swz<L::NC>(row)) << 4) + 8 * (ti & 1);
      }
      auto tr_operand = [&](const char* tile, int t, int db) {
        const char* base = tile + t * 16 * L::RB;
        const u32x2 lo = ld8_tr(base + (tb[0] ^ (db << 6)));
        const u32x2 hi = ld8_tr(base + (tb[1] ^ (db << 6)));
        return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
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

      // dV_j += P^T dO_i and dK_j += dS^T Q_i for the tile in stage st with its
      // fragments in slot fs: lane = feature column, register = key row
      auto grad_step = [&](int st, int fs) {
        const char* fb = smem + fs * L::F_BYTES + f_lane;
        const char* sb_ = stage_ptr(st);
        bf16x8 pb[2], sbf[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          pb[t] = as_bf16x8(ld16(fb + t * 1024));
          sbf[t] = as_bf16x8(ld16(fb + (2 + t) * 1024));
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < L::NDB; ++db) {
            dv[db] = mfma32(pb[t], tr_operand(sb_ + L::G_OFF, t, db), dv[db]);
            dk[db] = mfma32(sbf[t], tr_operand(sb_ + L::Q_OFF, t, db), dk[db]);
          }
        sched_read_pairs_ahead<4 * L::NDB, 4, 4>();
      };

      int tgr = next_tile(it0);                        // the tile of the next gradient step
      int t1 = next_tile(tgr + 1);                     // the tiles copied next
      int t2 = next_tile(t1 + 1);
      copy_tile(tgr, 0);
      copy_tile(t1, 1);
      wait_vmem_le<L::COPIES>();
      barrier_keep_vmem();
      // phase p: the score waves' step p; here the gradients of step p-1 and the
      // copy of step p+2's tile, into stage (p+2) % 4 (last read in phase p-1)
      for (int p = 0; p < n; ++p) {
        copy_tile(t2, (p + 2) & (L::NSTAGE - 1));
        t2 = next_tile(t2 + 1);
        if (p >= 1) {
          // causal: a query tile wholly before this wave's keys has all-zero fragments
          if (!CAUSAL || tgr * kBQ + kBQ - 1 >= kw0) grad_step((p - 1) & (L::NSTAGE - 1), (p - 1) & 1);
          tgr = next_tile(tgr + 1);
        }
        // this wave's copies of step p+1's tile have landed (they complete in
        // issue order; step p+2's may still be in flight), and its reads are done
        wait_vmem_le<L::COPIES>();
        wait_lds_all();
        barrier_keep_vmem();
      }
      // the last tile's gradients (stage and fragment slot of step n-1)
      if (n > 0 && (!CAUSAL || tgr * kBQ + kBQ - 1 >= kw0)) grad_step((n - 1) & (L::NSTAGE - 1), (n - 1) & 1);
      wait_vmem_all();                                 // no copy may land after the block is done

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
}

// ---------------------------------------------------------------------------
// Query-block sweep: dQ_i, in the other loop order ([ZtF] "Which loop goes
// outside?"), so that each dQ row is summed in registers by one wave and
// written once, with no atomics and a fixed summation order.
//
// d = 64 and 128 (d = 256 runs bwd_dq_split_kernel below).  One workgroup of
// eight waves per (256-query block, b, h).  Each wave owns 32 query rows and
// keeps their Q and dO fragments (MFMA B operands), lse, D and the float32 dQ^T
// accumulator in registers for a sweep over key blocks of 64 keys -- causal: up
// to the block's last query; tiles a wave cannot see are skipped by that wave.
// Per key block j:
//   * K_j and V_j go HBM -> LDS by buffer_load ... lds (rows XOR-swizzled by
//     16-byte chunk).  K_j serves both products: row reads for S^T, and
//     transposing 8-byte reads (one feature per lane, keys in the k-slot order
//     of the dS fragments) for K_j^T.
//   * S^T = K_j Q^T and dP^T - D = V_j dO^T - D on MFMA put one query per lane,
//     so lse and D are per-lane constants (-D seeds the accumulator):
//     P^T = exp2(S^T c log2e - lse log2e) and dS^T = P^T * (dP^T - D) ([ZtF]
//     "The backward pass, derived").
//   * dQ^T += K_j^T dS^T with dS^T rounded to bf16 straight from registers.
// Epilogue: dQ = scale * dQ~, once, in the gradient dtype.
// ---------------------------------------------------------------------------
template <int D>
struct DqLayout {
  static_assert(D == 64 || D == 128, "d = 256 runs bwd_dq_split_kernel");
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WAVES_PER_SIMD = WAVES / 4;
  static constexpr int BR = 32 * WAVES;                // query rows per workgroup
  static constexpr int BC = 64;                        // keys per block
  static constexpr int NC = D / 8;                     // 16-byte chunks per K/V row
  static constexpr int RB = D * 2;                     // bytes per K/V row
  static constexpr int KST = BC * RB;                  // K (or V) tile, swizzled rows, unpadded
  static constexpr int STAGE = 2 * KST;
  static constexpr int NSTAGE = 2;                     // two steps unrolled over two stage arrays
  static constexpr int BYTES = NSTAGE * STAGE;
  static constexpr int NKB = BC / 32;
  static constexpr int NDB = D / 32;
  static constexpr int NDS = D / 16;
  static constexpr int KDMA = KST / 1024;              // 1 KiB DMA instructions per K (or V) tile
  static constexpr int KDMA_W = 2 * KDMA / WAVES;      // per wave: the first half of the waves load K, the rest V
  static_assert((2 * KDMA) % WAVES == 0 && KDMA % (WAVES / 2) == 0, "DMA split over the waves");
  static_assert(NC == 8 || NC >= 16, "swizzle assumes 8 or >= 16 chunks per row");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
  static constexpr int K_OFF = 0, V_OFF = KST;        // within a stage
};

// Block-sparse dQ sweep: the workgroup's 256 queries span two 128-query mask
// rows.  Both rows go into LDS bitmaps (bit c = key block c visible); the
// workgroup visits the key tiles that either row can see, and a wave computes
// only those its own row can see.
template <int D, bool CAUSAL, bool MASKED, int BAND>
__global__ __launch_bounds__(DqLayout<D>::THREADS)
__attribute__((amdgpu_waves_per_eu(DqLayout<D>::WAVES_PER_SIMD))) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Ln, const float* __restrict__ Dn,
    void* __restrict__ dQ, int Tq, int Tk, float scale, float cl2e, int nqb, int grad_f32,
    const uint8_t* __restrict__ bmask, int H, long long mask_hstride, int nmk, int wl, int wr,
    const int* __restrict__ cu, int nd, int bcausal) {
  using L = DqLayout<D>;
  constexpr int BC = L::BC;
  static_assert(kMaskBlock % BC == 0 && L::BR % kMaskBlock == 0 && L::BR <= 2 * kMaskBlock,
                "one or two mask rows, whole tiles per mask block");
  // One LDS array per pipeline stage (distinct alias scopes: reads of one stage
  // need not wait for the DMA in flight into the other).
  __shared__ __attribute__((aligned(1024))) char stage0[L::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[L::STAGE];
  auto stage_ptr = [&](int st) -> char* { return st == 0 ? stage0 : stage1; };

  // Plain causal: workgroup p of a head runs query block nqb-1-p, then block p
  // (the long block first, as in the forward), so every workgroup sweeps about
  // the same number of key blocks (uneven workgroups leave CUs waiting on the
  // dispatcher).  Otherwise one block per
  // workgroup, causal sweeps longest first.
  constexpr bool PAIRED = CAUSAL && !MASKED && BAND == 0;
  const int nblk = gridDim.x, wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int npb = PAIRED ? (nqb + 1) / 2 : nqb;     // workgroups per head
  const int bh = lin / npb;
  const int pidx = lin % npb;
  const int npass = (PAIRED && 2 * pidx + 1 < nqb) ? 2 : 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  // Every wave runs every block's barriers; the early exit below only skips the
  // epilogue.  A block's last step ends on a barrier after all its LDS reads, so
  // the next block's first DMA cannot overwrite a tile still in use.
  for (int pass = 0; pass < npass; ++pass) {
    const int qb = !CAUSAL ? pidx : (npass == 2 && pass == 1) ? pidx : nqb - 1 - pidx;
    const int q0 = qb * L::BR;
    const int qw = q0 + wave * 32;
    const int myq = qw + lq;

    const rsrc_t rq = make_rsrc(Q + qbase, (unsigned)Tq * D * 2u);
    const rsrc_t rg = make_rsrc(dO + qbase, (unsigned)Tq * D * 2u);
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
    if (CAUSAL) ntile = min(ntile, (min(q0 + L::BR, Tq) - 1) / BC + 1);
    int jfirst = 0;                                     // first key block any row of the block can see
    // BAND: this lane's keys klo .. khi; over the wave's rows, the keys every row
    // sees (w_lo .. w_hi) and those some row sees (wb_lo .. wb_hi)
    int klo = 0, khi = 0, w_lo = 0, w_hi = 0, wb_lo = 0, wb_hi = 0;
    if constexpr (BAND != 0) {
      const Band<BAND> band{wl, wr, cu, nd, bcausal};
      band.keys(myq, klo, khi);
      w_lo = band.lo(qw + 31);
      w_hi = band.hi(qw);
      wb_lo = band.lo(qw);
      wb_hi = band.hi(qw + 31);
      const int b_hi = band.hi(min(q0 + L::BR, Tq) - 1);
      ntile = min(ntile, b_hi < 0 ? 0 : b_hi / BC + 1);
      jfirst = max(0, band.lo(q0)) / BC;
    }

    // ---- K (waves 0-3) and V (waves 4-7): HBM -> LDS, swizzled.  Lane l of DMA
    // instruction g moves chunk s = 64 (g % KDMA) + l of the tile: row s / NC,
    // stored chunk s % NC, which holds source chunk (s % NC) ^ row_swz(row).  The
    // lane offsets do not change between tiles; the tile's start goes into a
    // buffer resource over rows k0 .. Tk-1 (scalar work only), so rows past Tk --
    // and whole tiles past the end -- read as zeros.
    const uint16_t* const kv_src = wave < L::WAVES / 2 ? K : V;
    unsigned kvoff[L::KDMA_W];
#pragma unroll
    for (int i = 0; i < L::KDMA_W; ++i) {
      const int s = ((wave * L::KDMA_W + i) % L::KDMA) * 64 + lane;
      const int row = s / L::NC, cp = s % L::NC;
      kvoff[i] = (unsigned)(row * D + (cp ^ row_swz<L::NC>(row)) * 8) * 2u;
    }
    const unsigned* const kvo = kvoff;   // (the host compiler drops a kernel whose lambdas index a captured array)
    auto kv_dma = [&](int k0, int st) {
      const int rows = Tk - k0;
      const unsigned nbytes = rows > 0 ? (unsigned)rows * D * 2u : 0u;
      const uint16_t* const src = kv_src + kbase + (size_t)(k0 < Tk ? k0 : 0) * D;
      const rsrc_t r = make_rsrc(src, nbytes);
#pragma unroll
      for (int i = 0; i < L::KDMA_W; ++i) {
        const int g = wave * L::KDMA_W + i;            // 0 .. 2 KDMA - 1; V's follow K's in the stage
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(stage_ptr(st) + g * 1024), 16, kvo[i], 0, 0, 0);
      }
    };
    // per-lane K/V read offset for k-step ds: chunk (2 ds + hf) ^ swz of row lq
    const int swz_l = row_swz<L::NC>(lq);
    const int kbase_lane = lq * D * 2 + (((swz_l >> 1) << 5) | ((hf ^ (swz_l & 1)) << 4));

    // ---- K^T operand (A of dQ^T += K^T dS^T): lane l, row feature 32 db + l % 32,
    // elements = keys 16t + 4hf + 0..3 and 16t + 8 + 4hf + 0..3 of key block kb.
    // Each half comes from one transposing read in which lane 16g + 4e + j
    // addresses key row 4(g/2) + e (+ 8 for the second half) and features
    // 16(g%2) + 4j .. +3; tb[sec] is that offset for kb = t = db = 0.
    const int tg = lane >> 4, ti = lane & 15;
    int tb[2];
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int row = 8 * sec + 4 * (tg >> 1) + (ti >> 2);
      const int c = 2 * (tg & 1) + ((ti & 3) >> 1);
      tb[sec] = row * L::RB + ((c ^ row_swz<L::NC>(row)) << 4) + 8 * (ti & 1);
    }

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
    const bool has_b = L::BR == 2 * kMaskBlock && mr + 1 < (Tq + kMaskBlock - 1) / kMaskBlock;
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
    const int j0 = next_tile(jfirst);
    kv_dma(first_row(j0), 0);
    wait_vmem_all();
    __syncthreads();

    // tile j in stage ST; tile jc is copied into the other stage SC
    auto step = [&](int j, int ST, int jc, int SC) {
      // the mask test comes before the loads of block jn: a branch between those
      // loads and the reads of stage ST would make the compiler wait for the loads
      const bool sees = wave_sees(j);
      kv_dma(first_row(jc), SC);
      const int kt0 = j * BC;
      const bool in_band = BAND == 0 || (kt0 <= wb_hi && kt0 + BC - 1 >= wb_lo);
      if ((!CAUSAL || kt0 <= qw + 31) && sees && in_band) {   // some key of the block is visible to this wave
        const bool edge = (CAUSAL && kt0 + BC - 1 > qw) || (kt0 + BC > Tk) ||
                          (BAND != 0 && !(kt0 >= w_lo && kt0 + BC - 1 <= w_hi));
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
            ka[ds] = as_bf16x8(ld16(stage_ptr(ST) + L::K_OFF + off));
            va[ds] = as_bf16x8(ld16(stage_ptr(ST) + L::V_OFF + off));
          }
#pragma unroll
          for (int ds = 0; ds < L::NDS; ++ds) {
            s = mfma32(ka[ds], qf[ds], s);
            dp = mfma32(va[ds], gf[ds], dp);
          }
          // ten MFMAs of look-ahead (all eight at d = 64): -1.5% at d = 64, no
          // loss at 128
          sched_reads_ahead<2 * L::NDS, 2 * L::NDS, 10>();
          // K^T operands of the dQ product, read now so that their latency hides
          // behind the softmax: both k-steps at d = 64, k-step t = 0 only at d = 128
          // (all of them at once would spill there)
          const char* ks = stage_ptr(ST) + L::K_OFF + kb * 32 * L::RB;
          bf16x8 ta[2][L::NDB];
#pragma unroll
          for (int db = 0; db < L::NDB; ++db) {
            const u32x2 lo = ld8_tr(ks + (tb[0] ^ (db << 6)));
            const u32x2 hi = ld8_tr(ks + (tb[1] ^ (db << 6)));
            ta[0][db] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
          }
          if constexpr (D == 64) {
#pragma unroll
            for (int db = 0; db < L::NDB; ++db) {
              const u32x2 lo = ld8_tr(ks + 16 * L::RB + (tb[0] ^ (db << 6)));
              const u32x2 hi = ld8_tr(ks + 16 * L::RB + (tb[1] ^ (db << 6)));
              ta[1][db] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
          }
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(s[r], cl2e, lnq));
          if (edge) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
              if (key >= Tk || (CAUSAL && key > myq) || (BAND != 0 && (key < klo || key > khi))) p[r] = 0.f;
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
          // dQ^T += K_j^T dS^T: lane = query column, register = feature row (at
          // d = 128 the operands of k-step t = 1 are read here)
          if constexpr (D != 64) {
#pragma unroll
            for (int db = 0; db < L::NDB; ++db) {
              const u32x2 lo = ld8_tr(ks + 16 * L::RB + (tb[0] ^ (db << 6)));
              const u32x2 hi = ld8_tr(ks + 16 * L::RB + (tb[1] ^ (db << 6)));
              ta[1][db] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
          }
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int db = 0; db < L::NDB; ++db) dq[db] = mfma32(ta[t][db], sf[t], dq[db]);
        }
      }
      wait_vmem_all();
      __syncthreads();
    };

    // two steps per iteration, so that every stage offset is a constant
    if constexpr (MASKED) {
      for (int j = j0; j < ntile;) {
        int jn = next_tile(j + 1);
        step(j, 0, jn, 1);
        j = jn;
        if (j >= ntile) break;
        jn = next_tile(j + 1);
        step(j, 1, jn, 0);
        j = jn;
      }
    } else {
      for (int j = j0; j < ntile; j += 2) {
        step(j, 0, j + 1, 1);
        if (j + 1 < ntile) step(j + 1, 1, j + 2, 0);
      }
    }

    if (myq >= Tq) continue;
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
}

// ---------------------------------------------------------------------------
// Query-block sweep for d = 256 in two roles (bwd_dq_split_kernel).
//
// With one wave per query slice, the Q and dO fragments (128 registers per
// lane), the dQ^T accumulator (128) and the S/dP accumulators oversubscribe a
// wave's registers, and the compiler shuttles the accumulator between AGPRs and
// VGPRs around every dQ product.  Here a workgroup of eight waves covers 128
// queries, two waves per 32-query slice and per SIMD:
//   * score wave w (0-3) keeps slice w's Q and dO fragments, lse and D, forms
//     S^T = K_j Q^T and dP^T - D, then P^T and dS^T ([ZtF] "The backward pass,
//     derived"), and hands dS^T on through LDS as two MFMA fragments;
//   * gradient wave 4+w keeps slice w's dQ^T accumulator and trails its score
//     wave by one key block: dQ^T += K_j^T dS^T, K_j^T by transposing reads from
//     the same K tile.  The gradient waves also issue the copies.
// K_j and V_j go HBM -> LDS by buffer_load ... lds (inline assembly, unseen by
// the compiler) two blocks ahead into a ring of four stages; one bare barrier
// per phase.  Each slice's arithmetic, and the order of its dQ sums, are those
// of one wave of bwd_dq_kernel; against the one-role form of this sweep at
// d = 256 that it replaced, the results were the same bits.
// ---------------------------------------------------------------------------
template <int D>
struct DqsLayout {
  static constexpr int BR = 128;                       // query rows per workgroup (4 slices)
  static constexpr int BC = 32;                        // keys per block
  static constexpr int NC = D / 8;
  static constexpr int RB = D * 2;
  static constexpr int KST = BC * RB;                  // K (or V) tile, swizzled rows
  static constexpr int STAGE = 2 * KST;
  static constexpr int NSTAGE = 4;
  static constexpr int F_OFF = NSTAGE * STAGE;         // dS^T fragments: 2 KiB per score wave, two slots
  static constexpr int F_SLOT = 4 * 2048;
  static constexpr int BYTES = F_OFF + 2 * F_SLOT;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int COPIES = STAGE / 1024 / 4;      // 1 KiB copies per gradient wave and block
  static constexpr int K_OFF = 0, V_OFF = KST;
  static_assert(NC >= 16 && STAGE % 1024 == 0 && COPIES <= 15, "layout");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
  static_assert(BR == kMaskBlock, "one mask row per workgroup");
};

template <int D, bool CAUSAL, bool MASKED, int BAND>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Ln, const float* __restrict__ Dn,
    void* __restrict__ dQ, int Tq, int Tk, float scale, float cl2e, int nqb, int grad_f32,
    const uint8_t* __restrict__ bmask, int H, long long mask_hstride, int nmk, int wl, int wr,
    const int* __restrict__ cu, int nd, int bcausal) {
  using L = DqsLayout<D>;
  constexpr int BC = L::BC;
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
  auto stage_ptr = [&](int st) { return smem + st * L::STAGE; };

  constexpr bool PAIRED = CAUSAL && !MASKED && BAND == 0;
  const int nblk = gridDim.x, wid = blockIdx.x;
  const int lin = (nblk % 8 == 0) ? (wid % 8) * (nblk / 8) + wid / 8 : wid;
  const int npb = PAIRED ? (nqb + 1) / 2 : nqb;     // workgroups per head
  const int bh = lin / npb;
  const int pidx = lin % npb;
  const int npass = (PAIRED && 2 * pidx + 1 < nqb) ? 2 : 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const int ws = wave & 3;                             // query slice (score wave ws, gradient wave 4+ws)
  const size_t qbase = (size_t)bh * Tq * D, kbase = (size_t)bh * Tk * D;
  for (int pass = 0; pass < npass; ++pass) {
    if (pass > 0) {
      // the previous block's last reads are done before its stages are reused
      wait_lds_all();
      barrier_keep_vmem();
    }
    const int qb = !CAUSAL ? pidx : (npass == 2 && pass == 1) ? pidx : nqb - 1 - pidx;
    const int q0 = qb * L::BR;
    const int qw = q0 + ws * 32;
    const int myq = qw + lq;

    int ntile = (Tk + BC - 1) / BC;
    if (CAUSAL) ntile = min(ntile, (min(q0 + L::BR, Tq) - 1) / BC + 1);
    int jfirst = 0;
    int klo = 0, khi = 0, w_lo = 0, w_hi = 0, wb_lo = 0, wb_hi = 0;
    if constexpr (BAND != 0) {
      const Band<BAND> band{wl, wr, cu, nd, bcausal};
      band.keys(myq, klo, khi);
      w_lo = band.lo(qw + 31);
      w_hi = band.hi(qw);
      wb_lo = band.lo(qw);
      wb_hi = band.hi(qw + 31);
      const int b_hi = band.hi(min(q0 + L::BR, Tq) - 1);
      ntile = min(ntile, b_hi < 0 ? 0 : b_hi / BC + 1);
      jfirst = max(0, band.lo(q0)) / BC;
    }
    // visible key blocks: bit c of word w of the block's mask row = key block 64w + c kept
    const int nvw = (nmk + 63) >> 6;
    const uint8_t* mrow = MASKED ? bmask + (long long)(bh % H) * mask_hstride + (long long)(q0 / kMaskBlock) * nmk
                                 : nullptr;
    int cw = -1;
    unsigned long long ca = 0;
    auto word = [&](int w) {
      if (w != cw) {
        cw = w;
        ca = mask_word(mrow, 1, nmk, w, lane);
      }
      return ca;
    };
    auto next_tile = [&](int j) {                     // first visible block >= j, ntile if none
      if constexpr (MASKED) {
        if (j >= ntile) return ntile;
        const int c = j * BC / kMaskBlock;
        int w = c >> 6;
        unsigned long long bits = word(w) & (~0ull << (c & 63));
        while (bits == 0) {
          if (++w >= nvw) return ntile;
          bits = word(w);
        }
        const int c2 = w * 64 + (int)__builtin_ctzll(bits);
        return c2 == c ? j : min(ntile, c2 * (kMaskBlock / BC));
      } else {
        return j;
      }
    };
    // the tile's work for this slice: some key of the block visible to some row
    auto visible = [&](int j) {
      const int kt0 = j * BC;
      const bool in_band = BAND == 0 || (kt0 <= wb_hi && kt0 + BC - 1 >= wb_lo);
      return (!CAUSAL || kt0 <= qw + 31) && in_band;
    };
    const int j0 = next_tile(jfirst);

    if (wave < 4) {
      // ============================ score waves ============================
      const rsrc_t rq = make_rsrc(Q + qbase, (unsigned)Tq * D * 2u);
      const rsrc_t rg = make_rsrc(dO + qbase, (unsigned)Tq * D * 2u);
      const rsrc_t rl = make_rsrc(Ln + (size_t)bh * Tq, (unsigned)Tq * 4u);
      const rsrc_t rd = make_rsrc(Dn + (size_t)bh * Tq, (unsigned)Tq * 4u);
      bf16x8 qf[L::NDS], gf[L::NDS];
#pragma unroll
      for (int ds = 0; ds < L::NDS; ++ds) {
        const unsigned off = ((unsigned)myq * D + ds * 16 + 8 * hf) * 2u;
        qf[ds] = as_bf16x8(bload16(rq, off));
        gf[ds] = as_bf16x8(bload16(rg, off));
      }
      const float lnq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, myq * 4, 0, 0));
      const float dnq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, myq * 4, 0, 0));
      // per-lane K/V read offset for k-step ds: chunk (2 ds + hf) ^ swz of row lq
      const int swz_l = row_swz<L::NC>(lq);
      const int kbase_lane = lq * D * 2 + (((swz_l >> 1) << 5) | ((hf ^ (swz_l & 1)) << 4));
      barrier_keep_vmem();
      int p = 0;
      for (int j = j0; j < ntile; ++p) {
        const int jn = next_tile(j + 1);
        if (visible(j)) {
          const int kt0 = j * BC;
          const bool edge = (CAUSAL && kt0 + BC - 1 > qw) || (kt0 + BC > Tk) ||
                            (BAND != 0 && !(kt0 >= w_lo && kt0 + BC - 1 <= w_hi));
          const char* sb_ = stage_ptr(p & (L::NSTAGE - 1));
          // S^T and dP^T - D for the block's 32 keys: register r = key kt0 + 8(r/4)+4hf+r%4, lane = query
          f32x16 s, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[r] = 0.f;
            dp[r] = dnq;
          }
#pragma unroll
          for (int ds = 0; ds < L::NDS; ++ds) {
            const int off = kbase_lane ^ (ds << 5);
            s = mfma32(as_bf16x8(ld16(sb_ + L::K_OFF + off)), qf[ds], s);
            dp = mfma32(as_bf16x8(ld16(sb_ + L::V_OFF + off)), gf[ds], dp);
          }
          sched_reads_ahead<2 * L::NDS, 2 * L::NDS, 10>();
          float pr[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(__builtin_fmaf(s[r], cl2e, lnq));
          if (edge) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kt0 + 8 * (r >> 2) + 4 * hf + (r & 3);
              if (key >= Tk || (CAUSAL && key > myq) || (BAND != 0 && (key < klo || key > khi))) pr[r] = 0.f;
            }
          }
          char* fb = smem + L::F_OFF + (p & 1) * L::F_SLOT + ws * 2048 + lane * 16;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * t + 2 * e;
              w[e] = pack_bf16(pr[r] * dp[r], pr[r + 1] * dp[r + 1]);
            }
            st16(fb + t * 1024, w);
          }
        }
        // the fragments are complete, and so are this step's reads of the stage
        wait_lds_all();
        barrier_keep_vmem();
        j = jn;
      }
    } else {
      // =========================== gradient waves ==========================
      // Copies: waves 4-5 move K_j, waves 6-7 V_j; lane l of copy g (0 .. 2 COPIES
      // - 1 over the tensor's two waves) moves chunk s = 64 g + l of the tile: row
      // s / NC, stored at chunk s % NC, which holds source chunk (s % NC) ^
      // row_swz(row).  A block index past the sweep starts at row Tk: zeros.
      const int gw = wave - 4;
      const uint16_t* const src = gw >= 2 ? V : K;
      unsigned coff[L::COPIES];
#pragma unroll
      for (int i = 0; i < L::COPIES; ++i) {
        const int sidx = ((gw & 1) * L::COPIES + i) * 64 + lane;
        const int row = sidx / L::NC, cp = sidx % L::NC;
        coff[i] = (unsigned)(row * D + (cp ^ row_swz<L::NC>(row)) * 8) * 2u;
      }
      const unsigned* const co = coff;   // (the host compiler drops a kernel whose lambdas index a captured array)
      const unsigned lds0 = (unsigned)(size_t)smem;
      const unsigned c_dst = (gw >= 2 ? L::V_OFF : L::K_OFF) + (gw & 1) * L::COPIES * 1024;
      auto first_row = [&](int j) { return j < ntile ? j * BC : Tk; };
      auto copy_tile = [&](int j, int st) {
        const int k0 = first_row(j);
        const int rows = Tk - k0;
        const u32x4 r = raw_rsrc(src + kbase + (size_t)(k0 < Tk ? k0 : 0) * D, rows > 0 ? (unsigned)rows * D * 2u : 0u);
        const unsigned base = lds0 + (unsigned)st * L::STAGE + c_dst;
#pragma unroll
        for (int i = 0; i < L::COPIES; ++i) dma16_unseen(r, co[i], base + i * 1024);
      };
      // K^T operand (A of dQ^T += K^T dS^T): lane l, row feature 32 db + l % 32,
      // elements = keys 16t + 4hf + 0..3 and 16t + 8 + 4hf + 0..3, as in bwd_dq_kernel
      const int tg = lane >> 4, ti = lane & 15;
      int tb[2];
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int row = 8 * sec + 4 * (tg >> 1) + (ti >> 2);
        const int c = 2 * (tg & 1) + ((ti & 3) >> 1);
        tb[sec] = row * L::RB + ((c ^ row_swz<L::NC>(row)) << 4) + 8 * (ti & 1);
      }
      f32x16 dq[L::NDB];
#pragma unroll
      for (int db = 0; db < L::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;
      auto grad_step = [&](int st, int fs) {
        const char* fb = smem + L::F_OFF + fs * L::F_SLOT + ws * 2048 + lane * 16;
        const bf16x8 sf0 = as_bf16x8(ld16(fb)), sf1 = as_bf16x8(ld16(fb + 1024));
        const char* ks = stage_ptr(st) + L::K_OFF;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < L::NDB; ++db) {
            const u32x2 lo = ld8_tr(ks + 16 * t * L::RB + (tb[0] ^ (db << 6)));
            const u32x2 hi = ld8_tr(ks + 16 * t * L::RB + (tb[1] ^ (db << 6)));
            dq[db] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), t ? sf1 : sf0, dq[db]);
          }
        sched_read_pairs_ahead<2 * L::NDB, 4, 2>();
      };
      int jc1 = next_tile(j0 + 1);
      int jc2 = next_tile(jc1 + 1);
      copy_tile(j0, 0);
      copy_tile(jc1, 1);
      wait_vmem_le<L::COPIES>();
      barrier_keep_vmem();
      int p = 0, jprev = -1;
      for (int j = j0; j < ntile; ++p) {
        copy_tile(jc2, (p + 2) & (L::NSTAGE - 1));
        jc2 = next_tile(jc2 + 1);
        if (jprev >= 0 && visible(jprev)) grad_step((p - 1) & (L::NSTAGE - 1), (p - 1) & 1);
        jprev = j;
        j = next_tile(j + 1);
        // this wave's copies of the next block have landed (they complete in issue
        // order), and its reads of the stages are done
        wait_vmem_le<L::COPIES>();
        wait_lds_all();
        barrier_keep_vmem();
      }
      if (jprev >= 0 && visible(jprev)) grad_step((p - 1) & (L::NSTAGE - 1), (p - 1) & 1);
      wait_vmem_all();                                 // no copy may land after the block is done

      if (myq >= Tq) continue;
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
  }
}

template <int D>
int bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse, void* dQ,
        void* dK, void* dV, int B, int H, int Tq, int Tk, float scale, int causal, int o_f32, int grad_f32,
        void* workspace, int phases, hipStream_t stream, const uint8_t* bmask, int mask_heads, int band, int wl,
        int wr, const int* cu, int nd) {
  // query blocks of the dQ sweep: 256 rows (one role), 128 at d = 256 (two roles)
  constexpr int DQ_BR = [] {
    if constexpr (D == 256) return DqsLayout<D>::BR;
    else return DqLayout<D>::BR;
  }();
  const long long rows = (long long)B * H * Tq;
  const int nkb = (Tk + kBKC - 1) / kBKC;
  const long long nblk = (long long)nkb * B * H;
  const int nqb = (Tq + DQ_BR - 1) / DQ_BR;
  const long long nqblk = (long long)nqb * B * H;
  constexpr int RPB = 256 / (D / 8);           // rows per row-terms block
  const long long nrb = (rows + RPB - 1) / RPB;
  if (nblk > 0x7fffffffLL || nqblk > 0x7fffffffLL || nrb > 0x7fffffffLL) return FA_ERR_SHAPE;
  const float cl2e = scale * kLog2e;
  auto q = static_cast<const uint16_t*>(Q);
  auto k = static_cast<const uint16_t*>(K);
  auto v = static_cast<const uint16_t*>(V);
  auto g = static_cast<const uint16_t*>(dO);
  // block mask [mask_heads][ceil(Tq/128)][ceil(Tk/128)]
  const int nmq = (Tq + kMaskBlock - 1) / kMaskBlock, nmk = (Tk + kMaskBlock - 1) / kMaskBlock;
  const long long mhs = mask_heads == 1 ? 0 : (long long)nmq * nmk;
  // both sweeps read the negated row terms: Dn at the workspace start, Ln after it
  float* Dn = static_cast<float*>(workspace);
  float* Ln = Dn + bwd_rows_padded(rows);
  if (phases & FA_BWD_PRE) {
    if (o_f32)
      hipLaunchKernelGGL((row_terms_kernel<D, true>), dim3((unsigned)nrb), dim3(256), 0, stream, g, O, lse, Dn, Ln,
                         rows);
    else
      hipLaunchKernelGGL((row_terms_kernel<D, false>), dim3((unsigned)nrb), dim3(256), 0, stream, g, O, lse, Dn, Ln,
                         rows);
  }
  if (phases & FA_BWD_MAIN) {
    // key-block sweep: 8 waves in two roles for d <= 128, 4 waves for d = 256
    constexpr int KV_THREADS = D == 256 ? 256 : 512;
    // plain causal, d = 128: key blocks p and nkb-1-p share a workgroup
    const bool paired = D == 128 && causal && !bmask && band == 0;
    const long long nkv = paired ? (long long)((nkb + 1) / 2) * B * H : nblk;
    auto kv = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)nkv), dim3(KV_THREADS), 0, stream, q, k, v, g, Ln, Dn, dK, dV, Tq,
                         Tk, scale, cl2e, nkb, grad_f32, bmask, H, mhs, nmk, wl, wr, cu, nd, causal);
    };
    if constexpr (D == 256) {
      if (band == 1) kv(bwd_kv_w4_kernel<D, false, false, 1>);
      else if (band == 2) kv(bwd_kv_w4_kernel<D, false, false, 2>);
      else if (bmask) {
        if (causal) kv(bwd_kv_w4_kernel<D, true, true, 0>);
        else kv(bwd_kv_w4_kernel<D, false, true, 0>);
      } else {
        if (causal) kv(bwd_kv_w4_kernel<D, true, false, 0>);
        else kv(bwd_kv_w4_kernel<D, false, false, 0>);
      }
    } else {
      if (band == 1) kv(bwd_kv_kernel<D, false, false, 1>);
      else if (band == 2) kv(bwd_kv_kernel<D, false, false, 2>);
      else if (bmask) {
        if (causal) kv(bwd_kv_kernel<D, true, true, 0>);
        else kv(bwd_kv_kernel<D, false, true, 0>);
      } else {
        if (causal) kv(bwd_kv_kernel<D, true, false, 0>);
        else kv(bwd_kv_kernel<D, false, false, 0>);
      }
    }
  }
  if (phases & FA_BWD_POST) {
    // plain causal: query blocks nqb-1-p and p share a workgroup
    const bool paired = causal && !bmask && band == 0;
    const long long ndq = paired ? (long long)((nqb + 1) / 2) * B * H : nqblk;
    // both kernels run eight waves per workgroup
    auto dqk = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)ndq), dim3(512), 0, stream, q, k, v, g, Ln, Dn, dQ, Tq, Tk, scale,
                         cl2e, nqb, grad_f32, bmask, H, mhs, nmk, wl, wr, cu, nd, causal);
    };
    auto dqs = dqk;
    if constexpr (D == 256) {
      if (band == 1) dqs(bwd_dq_split_kernel<D, false, false, 1>);
      else if (band == 2) dqs(bwd_dq_split_kernel<D, false, false, 2>);
      else if (bmask) {
        if (causal) dqs(bwd_dq_split_kernel<D, true, true, 0>);
        else dqs(bwd_dq_split_kernel<D, false, true, 0>);
      } else {
        if (causal) dqs(bwd_dq_split_kernel<D, true, false, 0>);
        else dqs(bwd_dq_split_kernel<D, false, false, 0>);
      }
    } else {
      static_assert(DqLayout<D>::THREADS == 512, "eight waves");
      if (band == 1) dqk(bwd_dq_kernel<D, false, false, 1>);
      else if (band == 2) dqk(bwd_dq_kernel<D, false, false, 2>);
      else if (bmask) {
        if (causal) dqk(bwd_dq_kernel<D, true, true, 0>);
        else dqk(bwd_dq_kernel<D, false, true, 0>);
      } else {
        if (causal) dqk(bwd_dq_kernel<D, true, false, 0>);
        else dqk(bwd_dq_kernel<D, false, false, 0>);
      }
    }
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

int launch_bwd_bf16(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                    void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d, float scale, int causal,
                    int o_f32, int grad_f32, void* workspace, int phases, hipStream_t stream, const uint8_t* bmask,
                    int mask_heads, int band, int wl, int wr, const int* cu, int nd) {
  switch (d) {
    case 64: return bwd<64>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream, bmask, mask_heads, band, wl, wr, cu, nd);
    case 128: return bwd<128>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream, bmask, mask_heads, band, wl, wr, cu, nd);
    case 256: return bwd<256>(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, scale, causal, o_f32, grad_f32, workspace, phases, stream, bmask, mask_heads, band, wl, wr, cu, nd);
    default: return FA_ERR_HEADDIM;
  }
}

}  // namespace fa
