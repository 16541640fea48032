// Device-side building blocks for the gfx950 attention kernels: vector types,
// MFMA wrappers, 16-byte loads/stores, bf16 packing and cross-half reductions.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l holds row l%32, k-slots 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k-slots 8*(l/32) .. +7
//   D (32 x 32): lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
// Only the pairing of A's and B's k-slots matters for a product, so a kernel
// may assign any key/feature order to the slots as long as both operands
// agree.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Buffer resource over [base, base + nbytes): loads at byte offsets at or past
// nbytes return zeros instead of touching memory (the raw-buffer range check),
// which replaces per-row bounds branches for ragged tails.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, unsigned byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
// The same buffer resource as four words, for inline assembly: base address
// (48 bits), stride 0, size in bytes, and the flags word make_rsrc uses.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, unsigned nbytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, nbytes, 0x00020000u};
}

// buffer_load_dword{,x4} ... lds written out in assembly, HBM -> LDS: lane l's
// 4 (16) bytes from byte offset voff of the resource land at LDS byte address
// lds + 4 l (16 l); lds is wave-uniform and goes through M0.  The compiler does
// not see these as LDS writes, so it adds no waits for them: the caller waits
// with wait_vmem_le / wait_vmem_all before a barrier that hands the data on.
// (M0 is reserved for the compiler, which sets it before each of its own uses;
// no kernel that uses these also issues the builtin LDS copies.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_unseen(const u32x4& rsrc, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4_unseen(const u32x4& rsrc, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives as its
// element e (e = 0..3) the 16-bit element i % 4 of the 8 bytes addressed by lane
// 4e + i / 4 of the group.  When the lanes of a group address four consecutive
// rows of a row-major tile (four lanes per row, 4 columns each), every lane gets
// one column of those four rows: the transposed operand of an MFMA.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ld8_tr(const void* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<void*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// NaN-propagating maxima (v_maximum3_f32 on gfx950: no canonicalising moves).
__device__ __forceinline__ float max2f(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3f(float a, float b, float c) { return max2f(max2f(a, b), c); }

// Round two floats to bf16 (nearest-even; one v_cvt_pk_bf16_f32) packed low|high.
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// Value of the other half-wave's lane (l ^ 32) combined with this lane's value.
__device__ __forceinline__ float half_swap_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A value the whole wave holds alike, as a scalar register (v_readfirstlane).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }


// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maxima): every vector
// memory load issued so far has returned.  Placed where a loop iteration has
// already consumed its loads, it tells the compiler's wait-count tracking that
// nothing is outstanding at the back edge.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt lgkmcnt(0): this wave's LDS (and scalar) accesses have completed.
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence.  __syncthreads() is a release fence
// plus s_barrier, and the fence waits for every vector-memory load still in
// flight -- LDS DMA included -- which would drain a prefetch meant to stay in
// flight across the barrier.  This is the bare s_barrier; the "memory" clobber
// keeps the compiler from moving memory accesses across it.  The caller makes
// what others must see complete first: its LDS writes (wait_lds_all) and the
// DMA loads that must have landed (wait_vmem_le / wait_vmem_all).
__device__ __forceinline__ void barrier_keep_vmem() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N), N <= 15: at most the N vector memory loads issued last are
// still outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N <= 15, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Low / high bf16 halves of two words, packed (word a -> low half, word b -> high
// half); one v_perm_b32 each (selector bytes 0-3 pick from a, 4-7 from b).
__device__ __forceinline__ unsigned lo_lo(unsigned a, unsigned b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ unsigned hi_hi(unsigned a, unsigned b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// acc + lo + hi of a packed bf16 pair, in float32 (v_dot2c_f32_bf16 against 1.0).
__device__ __forceinline__ float add_bf16_pair(unsigned pair, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

// Scheduling hint for a block of LDS operand reads feeding MFMAs, written
// reads-first: keep the first reads A MFMAs ahead (six by default), then issue
// one read per MFMA.  Without it the scheduler issues each read just before its
// MFMA, so every MFMA pair waits out a full LDS round trip.
// With R reads and M MFMAs (R >= M) the first R - M + A reads go ahead; A is
// capped at M (all reads first).
template <int M, int R = M, int A0 = 6>
__device__ __forceinline__ void sched_reads_ahead() {
  constexpr int A = A0 < M ? A0 : M;
  static_assert(M >= 6 && R >= M, "at least six MFMAs, no fewer reads than MFMAs");
  __builtin_amdgcn_sched_group_barrier(0x100, R - M + A, 0);   // DS reads
#pragma unroll
  for (int i = 0; i < M - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}

// The same for operands that take two reads each (transposing 8-byte reads),
// after E reads of other operands: the first E + 2 A reads go ahead, then two
// reads per MFMA.
template <int M, int A0 = 4, int E = 0>
__device__ __forceinline__ void sched_read_pairs_ahead() {
  constexpr int A = A0 < M ? A0 : M;
  __builtin_amdgcn_sched_group_barrier(0x100, E + 2 * A, 0);
#pragma unroll
  for (int i = 0; i < M - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}

// Bits 64w .. 64w+63 of a byte mask, as one 64-bit word that is the same in
// every lane (bit i set iff m[(64w + i) * stride] != 0; entries at or past n
// read as 0).  A ballot puts it straight into scalar registers: one load per
// lane, no LDS and no barrier.  Call it with the whole wave active.
__device__ __forceinline__ unsigned long long mask_word(const uint8_t* m, long long stride, int n, int w, int lane) {
  const int i = w * 64 + lane;
  return __ballot(i < n && m[(long long)i * stride] != 0);
}

// The document of position x in a packed sequence: the largest i < n with
// cu[i] <= x, for offsets cu[0] = 0 <= cu[1] <= ... <= cu[n] of n documents.
// Reads cu[0 .. n-1] only; works for a wave-uniform or a per-lane x.
__device__ __forceinline__ int doc_of(const int* cu, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// A band mask: query r sees the keys lo(r) .. hi(r) and key l is seen by the
// queries qlo(l) .. qhi(l), all four non-decreasing.  KIND 1 is a sliding
// window, r - wl <= l <= r + wr (an unbounded side arrives as a large number);
// KIND 2 the documents of a packed sequence with offsets cu[0 .. nd], r and l
// in one document and, when causal, l <= r.
template <int KIND>
struct Band {
  int wl, wr;
  const int* cu;
  int nd, causal;
  __device__ int lo(int r) const {
    if constexpr (KIND == 1) return r - wl;
    else return cu[doc_of(cu, nd, r)];
  }
  __device__ int hi(int r) const {
    if constexpr (KIND == 1) return r + wr;
    else return causal ? r : cu[doc_of(cu, nd, r) + 1] - 1;
  }
  __device__ int qlo(int l) const {
    if constexpr (KIND == 1) return l - wr;
    else return causal ? l : cu[doc_of(cu, nd, l)];
  }
  __device__ int qhi(int l) const {
    if constexpr (KIND == 1) return l + wl;
    else return cu[doc_of(cu, nd, l) + 1] - 1;
  }
  // both ends with one search: the keys of query r, the queries of key l
  __device__ void keys(int r, int& a, int& b) const {
    if constexpr (KIND == 1) {
      a = r - wl;
      b = r + wr;
    } else {
      const int i = doc_of(cu, nd, r);
      a = cu[i];
      b = causal ? r : cu[i + 1] - 1;
    }
  }
  __device__ void queries(int l, int& a, int& b) const {
    if constexpr (KIND == 1) {
      a = l - wr;
      b = l + wl;
    } else {
      const int i = doc_of(cu, nd, l);
      a = causal ? l : cu[i];
      b = cu[i + 1] - 1;
    }
  }
};

}  // namespace fa
