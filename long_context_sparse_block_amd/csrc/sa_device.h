// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Two floats -> packed bf16 pair (lo = a), round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// bf16 pair dot product accumulated in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(32x32 f32) += A(32x16 bf16) * B(16x32 bf16).
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// D(32x32 f32) = A(32x16 bf16) * B(16x32 bf16) (zero accumulator, an inline constant).
__device__ __forceinline__ f32x16 mfma32_z(u32x4 a, u32x4 b) {
  const f32x16 z = {};
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), z, 0, 0, 0);
}

// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16).  Lane l holds row l%16 of A
// and column l%16 of B at k = 8(l/16) .. 8(l/16)+7, and column l%16 of D at
// rows 4(l/16) .. 4(l/16)+3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014): advance by the
// golden-ratio increment, then the 64-bit finaliser.  Host and device: the
// library's host RNG entry points run this same code, so it can be checked
// without a GPU.
__host__ __device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Keys of the library's counter-based draws (its own convention: no page
// fixes a generator): key(seed, tag, a, b, c) = sm(sm(sm(sm(sm(seed) ^ tag) ^
// a) ^ b) ^ c), evaluated as a per-(seed, tag, a) prefix and a finishing step.
__host__ __device__ __forceinline__ uint64_t key_prefix(uint64_t seed, uint64_t tag, uint64_t a) {
  return splitmix64(splitmix64(splitmix64(seed) ^ tag) ^ a);
}
__host__ __device__ __forceinline__ uint64_t key_finish(uint64_t prefix, uint64_t b, uint64_t c) {
  return splitmix64(splitmix64(prefix ^ b) ^ c);
}
constexpr uint64_t kTagLiteral = 1, kTagRandom = 2;

// Literal flag of block j from its key prefix key_prefix(seed, 1, flag group):
// the high 32 bits of key(seed, 1, f, j, 0) below floor(p * 2^32).
__host__ __device__ __forceinline__ bool literal_draw(uint64_t prefix, uint64_t j, uint64_t threshold) {
  return (key_finish(prefix, j, 0) >> 32) < threshold;
}

// The min(r, n) distinct uniform draws from [0, n) of row i of group g ("BigBird"
// Sec. 2, G_R: r sampled key blocks per query block; distinct, as the Sec. 3
// sketch takes a permutation prefix): candidate k is ((h >> 32) n) >> 32 with
// h = key(seed, 2, g, i, k); repeats are skipped; at most 64 r candidates.
// Writes the accepted values in draw order to out[0 .. count) and returns count.
__host__ __device__ inline int32_t draw_distinct(uint64_t seed, uint64_t g, uint64_t i, int32_t n, int32_t r,
                                                 int32_t* out) {
  const int32_t want = r < n ? r : n;
  int32_t cnt = 0;
  if (want <= 0) return 0;
  const uint64_t prefix = key_prefix(seed, kTagRandom, g);
  for (int32_t k = 0; k < 64 * r && cnt < want; ++k) {
    const uint64_t h = key_finish(prefix, i, (uint64_t)k);
    const int32_t x = (int32_t)(((h >> 32) * (uint64_t)n) >> 32);
    bool seen = false;
    for (int32_t m = 0; m < cnt; ++m) seen |= (out[m] == x);
    if (!seen) out[cnt++] = x;
  }
  return cnt;
}

__device__ __forceinline__ int wave_lane() { return __lane_id(); }

// The lane id computed afresh where it is used (v_mbcnt in volatile asm): the
// compiler can neither merge it with an earlier copy nor hoist it, so it never
// holds a register across a loop (or spills one) for it.
__device__ __forceinline__ int fresh_lane() {
  int l = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
#endif
  return l;
}

// Target builtins are wrapped in plain (non-template) device functions: a
// kernel template that names them directly is not instantiated by the host
// pass, and its launch stub would be missing.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Value of x in lane `src` (wave-uniform result, no memory access).
__device__ __forceinline__ int readlane(int x, int src) { return __builtin_amdgcn_readlane(x, src); }

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float max_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// max / sum of x over lanes l and l ^ 16 (v_permlane16_swap exchanges rows of
// 16 lanes pairwise: row 0 <-> row 1, row 2 <-> row 3).
__device__ __forceinline__ float max_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Value of x in lane byte_addr / 4 (ds_bpermute: LDS crossbar, no LDS memory).
__device__ __forceinline__ float bperm(int byte_addr, float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(byte_addr, __float_as_int(x)));
}

// Sum over the 4 lanes of a quad (DPP quad permutes).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  return x;
}

// 16-byte global load issued as inline asm (sbase: wave-uniform base pointer,
// voff: per-lane byte offset).  The compiler does not count it, so the caller
// waits for it with vm_wait<n>() (n = vector memory operations issued after it
// that may stay outstanding) and then tie()s the result, which orders every use
// after the wait.
__device__ __forceinline__ u32x4 gload16(const void* sbase, uint32_t voff) {
  u32x4 r;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(r) : "v"(voff), "s"(sbase) : "memory");
#else
  r = u32x4{0u, 0u, 0u, 0u};
#endif
  return r;
}
template <int N>
__device__ __forceinline__ void vm_wait() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
#endif
}
__device__ __forceinline__ void tie(u32x4& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
}

// Direct global -> LDS copies (global_load_lds_dwordx4): each lane's 16 bytes
// from sbase + voff land at M0 + 16 * lane (M0 = wave-uniform LDS address).
// Issued as inline asm so the compiler does not track them: it would otherwise
// wait for every outstanding copy before any later LDS read, which serialises
// a multi-stage ring.  The caller orders them with explicit "s_waitcnt vmcnt"
// and a barrier.  The instruction offset is added to both the global and the
// LDS address.  M0 is restored, so code around the asm may keep using it; one
// wait state separates the M0 write from the copy (GFX9 M0 -> LDS-DMA hazard).
// The asm is device-only: kernel templates that use these helpers must still
// instantiate in the host pass.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
#endif
}
// Two copies 2048 bytes apart in both spaces (rows that are contiguous in
// global memory and in LDS).
__device__ __forceinline__ void dma16x2(const void* sbase, uint32_t voff, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:2048\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
#endif
}

// Four copies of 2048-byte-spaced pairs: copies at (off, lds), (off + 2048,
// lds + 2048), (off4k, lds + 4096), (off4k + 2048, lds + 6144), where off4k =
// off + 4096 (one M0 save / restore for the four).
__device__ __forceinline__ void dma16x4p(const void* sbase, uint32_t off, uint32_t off4k, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "global_load_lds_dwordx4 %1, %3 offset:2048\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:2048\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "v"(off4k), "s"(sbase), "s"(lds), "s"(lds + 4096u)
      : "memory");
#endif
}

// Four copies 1024 bytes apart in both spaces.
__device__ __forceinline__ void dma16x4(const void* sbase, uint32_t voff, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:1024\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:2048\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
#endif
}

// Slot of 16-byte chunk c of a row of D bf16 values in an LDS tile (rows of
// 2D bytes, stored back to back).  gfx950 reads LDS as 64 banks of 4 bytes:
// ds_read_b128 serves 16 lanes per cycle and ds_read_b64_tr_b16 32 lanes.  The
// XOR below makes both access patterns of the MFMA operands conflict-free:
// 16 consecutive rows read at one logical chunk (b128), and 4 consecutive rows
// (a multiple of 4 first) read at 4 consecutive chunks with both 8-byte halves
// (transpose reads).  At D = 128 a row fills all 16 bank groups of 16 bytes,
// so the 16 rows need 16 distinct slots; at D = 64 two rows share the 16
// groups, so the slots of the 8 rows of each parity must differ.  The pattern
// repeats every 16 rows.
template <int D>
__device__ __forceinline__ int lds_slot(int c, int row) {
  static_assert(D == 64 || D == 128, "row width");
  if constexpr (D == 128)
    return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  else
    return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
constexpr int kSlotPeriod = 16;  // rows after which lds_slot repeats

// Slot pattern for a tile that is only read by transpose reads (4 consecutive
// rows at 4 consecutive chunks): the row's two low bits spread the 4 rows over
// distinct groups of slots.  Repeats every 4 rows, so rows 8 apart share their
// offsets.
template <int D>
__device__ __forceinline__ int lds_slot_tr(int c, int row) {
  static_assert(D == 64 || D == 128, "row width");
  return c ^ ((row & 3) << (D == 128 ? 2 : 1));
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Keep a value live in registers at this point (forces pending loads of it to
// complete here).
__device__ __forceinline__ void keep(const u32x4& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}
__device__ __forceinline__ void keep(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}
__device__ __forceinline__ void keep(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

// Transpose read of 4 x 16-bit values: within each group of 16 lanes, lane i
// receives element (i % 4) of the 8-byte words read by lanes i/4, i/4 + 4,
// i/4 + 8 and i/4 + 12 of the group (in that order).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)lds);
  return __builtin_bit_cast(u32x2, v);
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 in order, so that
// every index is a compile-time constant (unrolled at the source level).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace sa

// Instruction-scheduling hint for the device pass: the next `n` instructions of
// the kind in `mask` (0x2 VALU, 0x8 MFMA, 0x100 LDS read) form one group of the
// pattern the scheduler must follow within the current basic block.
// SA_SCHED_BARRIER: no instruction is moved across this point.
#if defined(__HIP_DEVICE_COMPILE__)
#define SA_SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
#define SA_SCHED_BARRIER() __builtin_amdgcn_sched_barrier(0)
#else
#define SA_SCHED_GROUP(mask, n)
#define SA_SCHED_BARRIER()
#endif
