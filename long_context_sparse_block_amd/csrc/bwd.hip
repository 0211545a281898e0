// Gradients of block-sparse and offset attention (dq, dk, dv) from the saved
// row log-sum-exp.  With P = exp(scale q k^T - lse) over the allowed pairs,
// dO the upstream gradient and D_t = <dO_t, o_t>:
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
//     dQ = scale dS K,   dK = scale dS^T Q
// (masked pairs contribute nothing; grouped-query heads add into their K/V
// head).  Kernels:
//   * delta: D = rowsum(dO * O), fp32 (for the block-sparse bf16 kernels
//     stored with lse log2(e) as one pair per row);
//   * mask transpose: the CSR key-block lists -> per key block the ascending
//     list of query blocks that list it (CSC), one wave per column;
//   * block-sparse bf16: a dQ kernel over the CSR rows (one workgroup per
//     query block, a wave per 32 queries, S^T = K Q^T so each lane owns a
//     query) and a dK/dV kernel over chunks of the CSC columns (persistent
//     workgroups, a wave per 32 keys, S = Q K^T so each lane owns a key); all
//     five products on v_mfma_f32_32x32x16_bf16, P and dS fed from the
//     accumulators as B operands, the transposed A operands (K^T, Q^T, dO^T)
//     by ds_read_b64_tr_b16 from LDS, the 64-row tiles staged by direct
//     global -> LDS copies into two-slot rings;
//   * offsets bf16: four adjacent lanes per row (coalesced 64-byte segments),
//     16 rows per wave, distances four at a time;
//   * block-sparse fp32 and offsets fp32: one thread per row, plain fp32
//     arithmetic (exactness path).
#include <math.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <type_traits>

#include "sa_device.h"
#include "sa_host.h"


namespace {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const float* lse;
  float* delta;
  sa::f32x2* stat;  // block-sparse bf16: per row {lse log2(e) (+inf if empty), D}
  int64_t st[8][3];  // q k v o dout dq dk dv: batch, head, sequence strides (elements)
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  const int32_t* sched;  // per group, the rows in launch order (or NULL: ascending)
  int64_t col_capacity, row_capacity;
  int32_t B, H, H_kv, N, nb, G;
  int64_t mbs, mhs;
  int32_t causal;
  float scale, c2;  // c2 = scale * log2(e)
  int32_t noff;
  int32_t offs[SA_MAX_OFFSETS];
  // block-sparse dK/dV work list: columns (b, kvh, j) split into chunks of
  // `chunk` entries; pre[c] = first work item of column c (exclusive scan)
  int32_t* pre;
  float* acc;  // fp32 [2][B][H_kv][N][d]: partial dK, dV of split columns
  int32_t chunk;  // least entries per chunk
  int64_t slots;  // dK/dV workgroups resident on the GPU at once
};

enum { TQ = 0, TK = 1, TV = 2, TO = 3, TDO = 4, TDQ = 5, TDK = 6, TDV = 7 };

inline sa_status allow_lds(const void* kern, int bytes) {
  if (bytes <= 65536) return SA_OK;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return e == hipSuccess ? SA_OK : sa_host::record_hip_error(e, "hipFuncSetAttribute");
}

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  typedef uint16_t T;
};
template <>
struct Elem<false> {
  typedef float T;
};

// n consecutive elements -> floats (n a multiple of 8)
template <int n, bool BF16>
__device__ __forceinline__ void load_f(const typename Elem<BF16>::T* p, float* out) {
  if constexpr (BF16) {
#pragma unroll
    for (int x = 0; x < n; x += 8) {
      const sa::u32x4 w = *(const sa::u32x4*)(p + x);
#pragma unroll
      for (int j = 0; j < 4; ++j) out[x + 2 * j] = sa::bf16_lo(w[j]), out[x + 2 * j + 1] = sa::bf16_hi(w[j]);
    }
  } else {
#pragma unroll
    for (int x = 0; x < n; x += 4) {
      const sa::f32x4 w = *(const sa::f32x4*)(p + x);
      out[x] = w[0], out[x + 1] = w[1], out[x + 2] = w[2], out[x + 3] = w[3];
    }
  }
}

template <int n, bool BF16>
__device__ __forceinline__ void store_f(typename Elem<BF16>::T* p, const float* in) {
  if constexpr (BF16) {
#pragma unroll
    for (int x = 0; x < n; x += 8) {
      sa::u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = sa::pack_bf16x2(in[x + 2 * j], in[x + 2 * j + 1]);
      *(sa::u32x4*)(p + x) = w;
    }
  } else {
#pragma unroll
    for (int x = 0; x < n; x += 4) *(sa::f32x4*)(p + x) = sa::f32x4{in[x], in[x + 1], in[x + 2], in[x + 3]};
  }
}

// lse * log2(e), with +inf for an empty row (its weights are then exp2(-inf) = 0)
__device__ __forceinline__ float lse2_of(float lse) { return lse == -INFINITY ? INFINITY : lse * sa::kLog2e; }

// ---------------------------------------------------------------- delta ----
// D[b, h, t] = <dO_t, o_t>; D/8 lanes per row, 8 elements each.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void delta_kernel(BwdArgs a) {
  typedef typename Elem<BF16>::T T;
  constexpr int LPR = D / 8;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;  // over B * H * N
  const int part = threadIdx.x % LPR;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const bool live = row < rows;
  const int64_t rr = live ? row : 0;
  const int64_t b = rr / ((int64_t)a.H * a.N), h = (rr / a.N) % a.H, t = rr % a.N;
  const T* O = (const T*)a.o + b * a.st[TO][0] + h * a.st[TO][1] + t * a.st[TO][2] + 8 * part;
  const T* G = (const T*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1] + t * a.st[TDO][2] + 8 * part;
  float x[8], y[8];
  load_f<8, BF16>(O, x);
  load_f<8, BF16>(G, y);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s = fmaf(x[j], y[j], s);
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, LPR);
  if (live && part == 0) a.delta[rr] = s;
}

// ------------------------------------------------------- mask transpose ----
struct TrArgs {
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int32_t* col_ptr;
  int32_t* row_idx;
  int64_t col_capacity, row_capacity;
  int32_t G, nb;
};

// Does row r (its entries ascending) list block j?
__device__ __forceinline__ bool row_has(const TrArgs& t, int64_t r, int32_t j) {
  int64_t lo = t.row_ptr[r], hi = t.row_ptr[r + 1];
  lo = max((int64_t)0, min(lo, t.col_capacity));
  hi = max(lo, min(hi, t.col_capacity));
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    const int32_t c = t.col_idx[mid];
    if (c == j) return true;
    if (c < j)
      lo = mid + 1;
    else
      hi = mid;
  }
  return false;
}

// One wave per column (g, j): FILL = false counts the rows listing j into
// col_ptr[g * nb + j + 1]; FILL = true writes them ascending from col_ptr[g * nb + j].
template <bool FILL>
__global__ __launch_bounds__(256) void transpose_kernel(TrArgs t) {
  const int lane = threadIdx.x & 63;
  const int64_t col = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= (int64_t)t.G * t.nb) return;
  const int64_t g = col / t.nb;
  const int32_t j = (int32_t)(col % t.nb);
  int64_t pos = FILL ? t.col_ptr[col] : 0;
  for (int32_t i0 = 0; i0 < t.nb; i0 += 64) {
    const int32_t i = i0 + lane;
    const bool hit = i < t.nb && row_has(t, g * t.nb + i, j);
    const uint64_t m = __ballot(hit);
    if (FILL && hit) {
      const int64_t at = pos + __popcll(m & ((1ull << lane) - 1ull));
      if (at < t.row_capacity) t.row_idx[at] = i;
    }
    pos += __popcll(m);
  }
  if (!FILL && lane == 0) t.col_ptr[col + 1] = (int32_t)pos;
}

// Inclusive scan of col_ptr[1 .. n] in place (col_ptr[0] = 0), one workgroup.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* p, int64_t n) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0, p[0] = 0;
  __syncthreads();
  for (int64_t base = 0; base < n; base += 1024) {
    const int64_t i = base + threadIdx.x;
    int32_t v = i < n ? p[i + 1] : 0;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t add = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < n) p[i + 1] = part[threadIdx.x] + carry;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
}

// ------------------------------------------------- block-sparse helpers ----
// CSR entry range of row (g, i), clamped to the capacity.
__device__ __forceinline__ void row_range(const BwdArgs& a, int64_t g, int32_t i, int32_t& e0, int32_t& e1) {
  const int64_t r = g * a.nb + i;
  int64_t x = a.row_ptr[r], y = a.row_ptr[r + 1];
  x = max((int64_t)0, min(x, a.col_capacity));
  y = max(x, min(y, a.col_capacity));
  e0 = sa::uniform((int32_t)x), e1 = sa::uniform((int32_t)y);
}
__device__ __forceinline__ void col_range(const BwdArgs& a, int64_t g, int32_t j, int32_t& e0, int32_t& e1) {
  const int64_t c = g * a.nb + j;
  int64_t x = a.col_ptr[c], y = a.col_ptr[c + 1];
  x = max((int64_t)0, min(x, a.row_capacity));
  y = max(x, min(y, a.row_capacity));
  e0 = sa::uniform((int32_t)x), e1 = sa::uniform((int32_t)y);
}

// ----------------------------------------------------- block-sparse fp32 ---
// dq: one thread per query of query block i (BLK threads), keys in 64-key tiles.
template <int D, int BLK>
__global__ __launch_bounds__(BLK) void bsa_bwd_dq_f32(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float ksm[64][D];
  __shared__ __attribute__((aligned(16))) float vsm[64][D];
  const int tid = threadIdx.x;
  const int32_t bh = blockIdx.x / a.nb, i = blockIdx.x % a.nb;
  const int32_t b = bh / a.H, h = bh % a.H, kvh = h / (a.H / a.H_kv);
  const int64_t g = (int64_t)b * a.mbs + (int64_t)h * a.mhs;
  const int64_t t = (int64_t)i * BLK + tid;
  const float* Q = (const float*)a.q + b * a.st[TQ][0] + h * a.st[TQ][1];
  const float* K = (const float*)a.k + b * a.st[TK][0] + kvh * a.st[TK][1];
  const float* V = (const float*)a.v + b * a.st[TV][0] + kvh * a.st[TV][1];
  const float* G = (const float*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1];
  float* DQ = (float*)a.dq + b * a.st[TDQ][0] + h * a.st[TDQ][1];
  float qv[D], gv[D], acc[D];
  load_f<D, false>(Q + t * a.st[TQ][2], qv);
  load_f<D, false>(G + t * a.st[TDO][2], gv);
#pragma unroll
  for (int x = 0; x < D; ++x) acc[x] = 0.f;
  const int64_t row = ((int64_t)b * a.H + h) * a.N + t;
  const float l2 = lse2_of(a.lse[row]), dd = a.delta[row];
  int32_t e0, e1;
  row_range(a, g, i, e0, e1);
  for (int32_t e = e0; e < e1; ++e) {
    const int32_t kb = a.col_idx[e];
    if (kb < 0 || kb >= a.nb || (a.causal && kb > i)) continue;
    for (int s0 = 0; s0 < BLK; s0 += 64) {
      const int64_t key0 = (int64_t)kb * BLK + s0;
      __syncthreads();
      for (int u = tid; u < 64 * D / 4; u += BLK) {
        const int key = u / (D / 4), c = u % (D / 4);
        *(sa::f32x4*)&ksm[key][4 * c] = *(const sa::f32x4*)(K + (key0 + key) * a.st[TK][2] + 4 * c);
        *(sa::f32x4*)&vsm[key][4 * c] = *(const sa::f32x4*)(V + (key0 + key) * a.st[TV][2] + 4 * c);
      }
      __syncthreads();
      for (int kk = 0; kk < 64; ++kk) {
        if (a.causal && key0 + kk > t) break;
        float dot = 0.f, dp = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) dot = fmaf(qv[x], ksm[kk][x], dot), dp = fmaf(gv[x], vsm[kk][x], dp);
        const float p = exp2f(dot * a.c2 - l2);
        const float ds = p * (dp - dd);
#pragma unroll
        for (int x = 0; x < D; ++x) acc[x] = fmaf(ds, ksm[kk][x], acc[x]);
      }
    }
  }
#pragma unroll
  for (int x = 0; x < D; ++x) acc[x] *= a.scale;
  store_f<D, false>(DQ + t * a.st[TDQ][2], acc);
}

// dk, dv: one thread per key of key block j (BLK threads), over the q heads
// of the K/V head and the query blocks that list j, queries in 32-row tiles.
template <int D, int BLK>
__global__ __launch_bounds__(BLK) void bsa_bwd_dkdv_f32(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float qsm[32][D];
  __shared__ __attribute__((aligned(16))) float gsm[32][D];
  __shared__ float lsm[32], dsm[32];
  const int tid = threadIdx.x;
  const int32_t bk = blockIdx.x / a.nb, j = blockIdx.x % a.nb;
  const int32_t b = bk / a.H_kv, kvh = bk % a.H_kv, rep = a.H / a.H_kv;
  const int64_t s = (int64_t)j * BLK + tid;
  const float* K = (const float*)a.k + b * a.st[TK][0] + kvh * a.st[TK][1];
  const float* V = (const float*)a.v + b * a.st[TV][0] + kvh * a.st[TV][1];
  float kv[D], vv[D], dk[D], dv[D];
  load_f<D, false>(K + s * a.st[TK][2], kv);
  load_f<D, false>(V + s * a.st[TV][2], vv);
#pragma unroll
  for (int x = 0; x < D; ++x) dk[x] = dv[x] = 0.f;
  for (int h = kvh * rep; h < (kvh + 1) * rep; ++h) {
    const int64_t g = (int64_t)b * a.mbs + (int64_t)h * a.mhs;
    const float* Q = (const float*)a.q + b * a.st[TQ][0] + h * a.st[TQ][1];
    const float* G = (const float*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1];
    const int64_t rowb = ((int64_t)b * a.H + h) * a.N;
    int32_t e0, e1;
    col_range(a, g, j, e0, e1);
    for (int32_t e = e0; e < e1; ++e) {
      const int32_t qb = a.row_idx[e];
      if (qb < 0 || qb >= a.nb || (a.causal && qb < j)) continue;
      for (int t0 = 0; t0 < BLK; t0 += 32) {
        const int64_t q0 = (int64_t)qb * BLK + t0;
        __syncthreads();
        for (int u = tid; u < 32 * D / 4; u += BLK) {
          const int r = u / (D / 4), c = u % (D / 4);
          *(sa::f32x4*)&qsm[r][4 * c] = *(const sa::f32x4*)(Q + (q0 + r) * a.st[TQ][2] + 4 * c);
          *(sa::f32x4*)&gsm[r][4 * c] = *(const sa::f32x4*)(G + (q0 + r) * a.st[TDO][2] + 4 * c);
        }
        if (tid < 32) lsm[tid] = lse2_of(a.lse[rowb + q0 + tid]), dsm[tid] = a.delta[rowb + q0 + tid];
        __syncthreads();
        for (int r = 0; r < 32; ++r) {
          if (a.causal && q0 + r < s) continue;
          float dot = 0.f, dp = 0.f;
#pragma unroll
          for (int x = 0; x < D; ++x) dot = fmaf(qsm[r][x], kv[x], dot), dp = fmaf(gsm[r][x], vv[x], dp);
          const float p = exp2f(dot * a.c2 - lsm[r]);
          const float ds = p * (dp - dsm[r]);
#pragma unroll
          for (int x = 0; x < D; ++x) dk[x] = fmaf(ds, qsm[r][x], dk[x]), dv[x] = fmaf(p, gsm[r][x], dv[x]);
        }
      }
    }
  }
#pragma unroll
  for (int x = 0; x < D; ++x) dk[x] *= a.scale;
  store_f<D, false>((float*)a.dk + b * a.st[TDK][0] + kvh * a.st[TDK][1] + s * a.st[TDK][2], dk);
  store_f<D, false>((float*)a.dv + b * a.st[TDV][0] + kvh * a.st[TDV][1] + s * a.st[TDV][2], dv);
}

// ----------------------------------------------------- block-sparse bf16 ---
// v_mfma_f32_32x32x16_bf16 layouts: A (32 x 16): lane l row l%32, k 8(l/32)..+8;
// B (16 x 32): lane l column l%32, k 8(l/32)..+8; C: lane l column l%32,
// rows 8(r/4) + 4(l/32) + r%4 for r < 16.  A product whose k index runs over
// the rows of a C tile takes, for k-step s (16 rows), the C entries
// r = 8s .. 8s+7 of the lane as its B operand; k slot 8(l/32) + e then stands
// for row 16s + 8(e/4) + 4(l/32) + e%4, and the matching A operand is read
// transposed from LDS with two ds_read_b64_tr_b16 (rows 16s + 4(l/32) + m and
// 16s + 8 + 4(l/32) + m).

// 16-byte chunk slot of a tile row in LDS: sa::lds_slot, conflict-free for
// both the row reads (ds_read_b128) and the transpose reads below.
template <int D>
__device__ __forceinline__ int bswz(int c, int row) { return sa::lds_slot<D>(c, row); }

template <int D>
struct TileLds {
  static constexpr int ROWB = 2 * D;
  // A operand of rows [r0, r0 + 32), d-chunks 2u + l/32 (16 d per k-step u)
  static __device__ __forceinline__ sa::u32x4 rows_a(const uint8_t* t, int r0, int u, int lane) {
    const int row = r0 + (lane & 31);
    return *(const sa::u32x4*)(t + row * ROWB + bswz<D>(2 * u + (lane >> 5), row) * 16);
  }
  // the same from an LDS byte address
  static __device__ __forceinline__ sa::u32x4 rows_a_lds(uint32_t t, int r0, int u, int lane) {
    const int row = r0 + (lane & 31);
    typedef __attribute__((address_space(3))) const sa::u32x4* lptr;
    return *(lptr)(uintptr_t)(t + row * ROWB + bswz<D>(2 * u + (lane >> 5), row) * 16);
  }
  // The slot pattern depends on a row's low four bits only, so for r0 a
  // multiple of 16 the reads above and below are a lane-constant byte offset
  // from t + r0 ROWB: a_off(u) for rows_a, tr_off(dt, ab) for the two reads
  // of rows_tr (ab = 0: rows 4(l/32) + m, ab = 1: 8 rows further).
  static __device__ __forceinline__ int a_off(int u, int lane) {
    const int row = lane & 31;
    return row * ROWB + bswz<D>(2 * u + (lane >> 5), row) * 16;
  }
  static __device__ __forceinline__ int tr_off(int dt, int ab, int lane) {
    const int grp = lane >> 4, p = lane & 15;
    const int d0 = 32 * dt + 16 * (grp & 1) + 4 * (p & 3);
    const int r = 4 * (grp >> 1) + (p >> 2) + 8 * ab;
    return r * ROWB + bswz<D>(d0 >> 3, r) * 16 + (d0 & 7) * 2;
  }
  static __device__ __forceinline__ sa::u32x4 at_a(const uint8_t* base, int off) {
    return *(const sa::u32x4*)(base + off);
  }
  static __device__ __forceinline__ sa::u32x4 at_tr(const uint8_t* base, int offa, int offb) {
    const sa::u32x2 x = sa::lds_read_tr16(base + offa);
    const sa::u32x2 y = sa::lds_read_tr16(base + offb);
    return sa::u32x4{x[0], x[1], y[0], y[1]};
  }
  // transposed A operand: d rows 32 dt + l%32, k = tile rows 16 s + 8(e/4) + 4(l/32) + e%4
  static __device__ __forceinline__ sa::u32x4 rows_tr(const uint8_t* t, int r0, int s, int dt, int lane) {
    const int grp = lane >> 4, p = lane & 15, h = grp >> 1;
    const int d0 = 32 * dt + 16 * (grp & 1) + 4 * (p & 3);  // first d of the lane's 8-byte word
    const int ra = r0 + 16 * s + 4 * h + (p >> 2), rb = ra + 8;
    const int ca = d0 >> 3, half = (d0 & 7) * 2;
    const sa::u32x2 x = sa::lds_read_tr16(t + ra * ROWB + bswz<D>(ca, ra) * 16 + half);
    const sa::u32x2 y = sa::lds_read_tr16(t + rb * ROWB + bswz<D>(ca, rb) * 16 + half);
    return sa::u32x4{x[0], x[1], y[0], y[1]};
  }
};

// Direct (DMA) copies of one 64-row bf16 tile into a swizzled LDS tile.  Wave
// w of NW issues JN copies of 64 16-byte chunks; chunk u = 64 (j NW + w) + lane
// of copy j is row u / CPR, slot u % CPR, and lane `lane` reads the global
// chunk that belongs in that slot.  Copy j reads RPC j rows further down and
// lands j NW KiB further into the tile; when RPC is a multiple of the slot
// pattern's period one per-lane source offset serves every copy, otherwise
// (RPC = 8: d = 128 with two waves) odd copies take a second offset.
template <int D, int NW>
struct TileDma {
  static constexpr int CPR = D / 8;
  static constexpr int JN = CPR / NW;         // copies per wave per tile
  static constexpr int RPC = NW * 64 / CPR;   // rows between a wave's copies
  static constexpr int TB = 64 * 2 * D;       // bytes of one tile
  static constexpr bool ODD = RPC % sa::kSlotPeriod != 0;
  static_assert(JN >= 1 && RPC % 8 == 0, "tile split");
  struct Off {
    uint32_t even, odd;
  };
  static __device__ __forceinline__ Off lane_off(int w, int lane, int64_t rs) {
    const int r0 = (64 * w + lane) / CPR, p = lane % CPR;
    const uint32_t row = (uint32_t)(r0 * rs * 2);
    Off o;
    o.even = row + 16u * (uint32_t)bswz<D>(p, r0);
    o.odd = ODD ? row + 16u * (uint32_t)bswz<D>(p, r0 + RPC) : o.even;
    return o;
  }
  static __device__ __forceinline__ void copy(const uint16_t* src, int64_t rs, Off off, uint32_t lds, int w) {
#pragma unroll
    for (int j = 0; j < JN; ++j)
      sa::dma16((const char*)src + (int64_t)j * RPC * rs * 2, (j & 1) ? off.odd : off.even, lds + (j * NW + w) * 1024);
  }
};

// Barrier that leaves outstanding direct copies in flight; ordering is by
// explicit "s_waitcnt vmcnt".
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Wait until at most c * J vector memory operations of this wave are
// outstanding (c in {0, 1}).
template <int J>
__device__ __forceinline__ void wait_units(int c) {
  if (c > 0)
    sa::vm_wait<J>();
  else
    sa::vm_wait<0>();
}

// pack C entries 8s .. 8s+7 into a bf16 B operand
__device__ __forceinline__ sa::u32x4 pack8(const float* x) {
  return sa::u32x4{sa::pack_bf16x2(x[0], x[1]), sa::pack_bf16x2(x[2], x[3]), sa::pack_bf16x2(x[4], x[5]),
                   sa::pack_bf16x2(x[6], x[7])};
}

// The two 32-row halves of a 64-row tile, one loop body: the causal mask of
// the diagonal tile is a wave-uniform branch inside it.  (A second copy of
// the loop for the diagonal tile made the compiler move the dK / dV
// accumulators between register sets around it on every tile.)
template <typename F>
__device__ __forceinline__ void bwd_tile(F& half) {
#pragma unroll 1
  for (int x = 0; x < 2; ++x) half(x);
}

// dq: one workgroup (BLK/32 waves) per query block, a wave per 32 queries.  The
// row's key blocks are walked in 64-row tiles of K and V, copied global -> LDS
// by direct loads into a ring of S slots: tile n + S - 1 is in flight while
// tile n is used.  Entries whose block is unusable (out of range, or after the
// query block when causal) load a safe tile and skip the arithmetic.
template <int D, int BLK, int S>
__global__ __launch_bounds__(2 * BLK) void bsa_bwd_dq_bf16(BwdArgs a) {
  using L = TileLds<D>;
  constexpr int NW = BLK / 32, NU = D / 16, NT = D / 32, SUBS = BLK / 64;
  using M = TileDma<D, NW>;
  constexpr int SLOT = 2 * M::TB;  // K tile, V tile
  constexpr int CP = 2 * M::JN;    // copies per wave per tile
  static_assert(S == 2 || S == 3, "ring slots");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = sa::uniform(tid >> 6), hl = lane >> 5;
  // blockIdx = pos * (B * H) + bh: with B * H a multiple of 8 every query
  // block of one head runs on the same XCD (the key blocks that neighbouring
  // query blocks share stay in one L2); pos is a launch position of the
  // head's mask group, longest row first when `sched` is given
  const int32_t BH = a.B * a.H;
  const int32_t bh = blockIdx.x % BH, pos = blockIdx.x / BH;
  const int32_t b = bh / a.H, h = bh % a.H, kvh = h / (a.H / a.H_kv);
  const int64_t g = (int64_t)b * a.mbs + (int64_t)h * a.mhs;
  const int32_t i = sa::uniform(a.sched ? a.sched[g * a.nb + pos] : pos);
  if (i < 0 || i >= a.nb) return;
  const int qoff = 32 * w + (lane & 31);           // this lane's query inside the block
  const int64_t tq = (int64_t)i * BLK + qoff;      // ... and in the sequence (C column)
  const uint16_t* Q = (const uint16_t*)a.q + b * a.st[TQ][0] + h * a.st[TQ][1];
  const uint16_t* K = (const uint16_t*)a.k + b * a.st[TK][0] + kvh * a.st[TK][1];
  const uint16_t* V = (const uint16_t*)a.v + b * a.st[TV][0] + kvh * a.st[TV][1];
  const uint16_t* G = (const uint16_t*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1];
  const int64_t ks2 = a.st[TK][2], vs2 = a.st[TV][2];
  sa::u32x4 qb[NU], gb[NU];  // B operands: column = query, k = d 16u + 8(l/32) ..
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    qb[u] = *(const sa::u32x4*)(Q + tq * a.st[TQ][2] + 16 * u + 8 * hl);
    gb[u] = *(const sa::u32x4*)(G + tq * a.st[TDO][2] + 16 * u + 8 * hl);
  }
  // the row statistics: D = <dO, o> (this lane holds d 16u + 8 hl .. + 7, the
  // other half in lane ^ 32) and lse in log2 units; stored for the dK/dV kernel
  const uint16_t* Ov = (const uint16_t*)a.o + b * a.st[TO][0] + h * a.st[TO][1];
  float dsum = 0.f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const sa::u32x4 ob = *(const sa::u32x4*)(Ov + tq * a.st[TO][2] + 16 * u + 8 * hl);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      dsum = __builtin_fmaf(sa::bf16_lo(ob[x]), sa::bf16_lo(gb[u][x]), dsum);
      dsum = __builtin_fmaf(sa::bf16_hi(ob[x]), sa::bf16_hi(gb[u][x]), dsum);
    }
  }
  const int64_t srow = ((int64_t)b * a.H + h) * a.N + tq;
  const float dd = sa::sum_xor32(dsum), l2 = lse2_of(a.lse[srow]);
  if (hl == 0) a.stat[srow] = sa::f32x2{l2, dd};
  sa::f32x16 acc[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) acc[dt] = sa::f32x16{};
  const typename M::Off offK = M::lane_off(w, lane, ks2), offV = M::lane_off(w, lane, vs2);
  const uint32_t ring = sa::lds_addr(smem);
  int aoff[NU], troff[NT][2];
#pragma unroll
  for (int u = 0; u < NU; ++u) aoff[u] = L::a_off(u, lane);
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) troff[dt][0] = L::tr_off(dt, 0, lane), troff[dt][1] = L::tr_off(dt, 1, lane);
  int32_t e0, e1;
  row_range(a, g, i, e0, e1);
  const int32_t limit = a.causal ? i + 1 : a.nb;  // usable key blocks are < limit
  bool first = true;
  for (int32_t base = e0; base < e1; base += 64) {
    const int cnt = min(64, e1 - base);
    const int32_t lst = lane < cnt ? a.col_idx[base + lane] : -1;  // entry base + x in lane x
    // the loads above complete here, before any copy is in flight
#pragma unroll
    for (int u = 0; u < NU; ++u) sa::keep(qb[u]), sa::keep(gb[u]);
    sa::keep(lst), sa::keep(l2), sa::keep(dd);
    if (!first) ring_barrier();  // every wave is done with the ring
    first = false;
    const int T = cnt * SUBS;
    auto tile_kb = [&](int m) -> int32_t {
      const int32_t kb = sa::readlane(lst, m / SUBS);
      return (uint32_t)kb < (uint32_t)limit ? kb : -1;
    };
    auto issue = [&](int m) {
      const int32_t kb = tile_kb(m);
      const int64_t r0 = (int64_t)(kb < 0 ? i : kb) * BLK + 64 * (m % SUBS);
      const uint32_t dst = ring + (m % S) * SLOT;
      M::copy(K + r0 * ks2, ks2, offK, dst, w);
      M::copy(V + r0 * vs2, vs2, offV, dst + M::TB, w);
    };
    issue(0);
    if (S > 2 && T > 1) issue(1);
    for (int n = 0; n < T; ++n) {
      wait_units<CP>(S > 2 && n + 1 < T);
      ring_barrier();
      if (n + S - 1 < T) issue(n + S - 1);
      const int32_t kb = tile_kb(n);
      if (kb < 0) continue;
      const uint8_t* ks = smem + (n % S) * SLOT;
      const uint8_t* vs = ks + M::TB;
      const int ksub = 64 * (n % SUBS);
      const bool diag = a.causal && kb == i;
      // The tile's two 32-key halves, software-pipelined inside the wave: the
      // S^T / dP^T MFMAs of half 1 run while the VALU turns half 0's S^T and
      // dP^T into dS^T, and dQ^T += K^T dS^T of half 0 runs while the VALU
      // works on half 1.  Operand reads go ahead of their MFMAs (scheduling
      // barriers and group patterns hold the order; the compiler counts the
      // reads in its waits).  The causal mask of the diagonal tile is applied
      // in a wave-uniform branch between the phases.
      constexpr int NA = 2 * NU;  // S^T and dP^T MFMAs of a half: m = 2u (K rows), 2u + 1 (V rows)
      constexpr int NC = 2 * NT;  // dQ^T MFMAs of a half: j = st NT + dt
      constexpr int RA = 3, RC = 2;
      sa::u32x4 abuf[2][NA], cbuf[2][NC];
      auto ard = [&](auto kt_, auto m) {
        constexpr int KT = decltype(kt_)::value, Mi = decltype(m)::value;
        if constexpr (Mi < NA)
          abuf[KT][Mi] = L::at_a(ks + 32 * KT * L::ROWB + ((Mi & 1) ? M::TB : 0), aoff[Mi >> 1]);
      };
      auto crd = [&](auto kt_, auto jj) {
        constexpr int KT = decltype(kt_)::value, J = decltype(jj)::value;
        if constexpr (J < NC)
          cbuf[KT][J] = L::at_tr(ks + (32 * KT + 16 * (J / NT)) * L::ROWB, troff[J % NT][0], troff[J % NT][1]);
      };
      using H0 = std::integral_constant<int, 0>;
      using H1 = std::integral_constant<int, 1>;
      auto sdp_mfma = [&](auto kt_, auto m, sa::f32x16& s_, sa::f32x16& dp_) {
        constexpr int KT = decltype(kt_)::value, Mi = decltype(m)::value;
        if constexpr (Mi == 1)
          dp_ = sa::mfma32_z(abuf[KT][Mi], gb[0]);
        else if constexpr (Mi & 1)
          dp_ = sa::mfma32(abuf[KT][Mi], gb[Mi >> 1], dp_);
        else if constexpr (Mi == 0)
          s_ = sa::mfma32_z(abuf[KT][Mi], qb[0]);
        else
          s_ = sa::mfma32(abuf[KT][Mi], qb[Mi >> 1], s_);
      };
      // dS^T of a half (unmasked)
      auto dsoft = [&](const sa::f32x16& s_, const sa::f32x16& dp_, float (&ds)[16]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = sa::fast_exp2(__builtin_fmaf(s_[r], a.c2, -l2)) * (dp_[r] - dd);
      };
      // keys after the query, on the diagonal tile only (a wave-uniform
      // branch, kept as one by the volatile asm); the lane's query less the
      // key offset 4 hl comes from a fresh lane id
      auto dmask = [&](float (&ds)[16], int kt) {
        if (diag) {
          asm volatile("" ::: "memory");
          const int fl = sa::fresh_lane();
          const int qd = 32 * w + (fl & 31) - 4 * (fl >> 5) - ksub - 32 * kt;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) > qd) ds[r] = 0.f;
        }
      };
      sa::f32x16 s0, dp0, s1, dp1;
      float ds0[16], ds1[16];
      // S^T, dP^T of half 0
      sa::static_for<0, RA>([&](auto m) { ard(H0{}, m); });
      sa::static_for<0, NA>([&](auto m) {
        constexpr int Mi = decltype(m)::value;
        SA_SCHED_BARRIER();
        sdp_mfma(H0{}, m, s0, dp0);
        ard(H0{}, std::integral_constant<int, Mi + RA>{});
      });
      SA_SCHED_BARRIER();
      // S^T, dP^T of half 1 beside dS^T of half 0
      sa::static_for<0, RA>([&](auto m) { ard(H1{}, m); });
      SA_SCHED_BARRIER();
      sa::static_for<0, NA>([&](auto m) {
        constexpr int Mi = decltype(m)::value;
        sdp_mfma(H1{}, m, s1, dp1);
        ard(H1{}, std::integral_constant<int, Mi + RA>{});
      });
      dsoft(s0, dp0, ds0);
      sa::static_for<0, NA>([&](auto m) {
        constexpr int Mi = decltype(m)::value;
        SA_SCHED_GROUP(0x008, 1);
        if constexpr (Mi + RA < NA) SA_SCHED_GROUP(0x100, 1);
        SA_SCHED_GROUP(0x002, 64 / NA);
      });
      SA_SCHED_GROUP(0x002, 64);
      SA_SCHED_BARRIER();
      dmask(ds0, 0);
      const sa::u32x4 bo0[2] = {pack8(ds0), pack8(ds0 + 8)};
      // dQ^T of half 0 beside dS^T of half 1
      sa::static_for<0, RC>([&](auto j) { crd(H0{}, j); });
      SA_SCHED_BARRIER();
      sa::static_for<0, NC>([&](auto jj) {
        constexpr int J = decltype(jj)::value;
        acc[J % NT] = sa::mfma32(cbuf[0][J], bo0[J / NT], acc[J % NT]);
        crd(H0{}, std::integral_constant<int, J + RC>{});
      });
      dsoft(s1, dp1, ds1);
      sa::static_for<0, NC>([&](auto jj) {
        constexpr int J = decltype(jj)::value;
        SA_SCHED_GROUP(0x008, 1);
        if constexpr (J + RC < NC) SA_SCHED_GROUP(0x100, 2);
        SA_SCHED_GROUP(0x002, 64 / NC);
      });
      SA_SCHED_GROUP(0x002, 64);
      SA_SCHED_BARRIER();
      dmask(ds1, 1);
      const sa::u32x4 bo1[2] = {pack8(ds1), pack8(ds1 + 8)};
      // dQ^T of half 1
      sa::static_for<0, RC>([&](auto j) { crd(H1{}, j); });
      sa::static_for<0, NC>([&](auto jj) {
        constexpr int J = decltype(jj)::value;
        SA_SCHED_BARRIER();
        acc[J % NT] = sa::mfma32(cbuf[1][J], bo1[J / NT], acc[J % NT]);
        crd(H1{}, std::integral_constant<int, J + RC>{});
      });
      SA_SCHED_BARRIER();
    }
  }
  // C rows of tile dt are d = 32 dt + 8(r/4) + 4(l/32) + r%4 of this lane's query
  uint16_t* DQ = (uint16_t*)a.dq + b * a.st[TDQ][0] + h * a.st[TDQ][1] + tq * a.st[TDQ][2];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const sa::f32x16& x = acc[dt];
      const int r = 4 * r4;
      const sa::u32x2 wv = {sa::pack_bf16x2(x[r] * a.scale, x[r + 1] * a.scale),
                            sa::pack_bf16x2(x[r + 2] * a.scale, x[r + 3] * a.scale)};
      *(sa::u32x2*)(DQ + 32 * dt + 8 * r4 + 4 * hl) = wv;
    }
}

// Column c = (b * H_kv + kvh) * nb + j of the dK/dV work: its entries are the
// transposed-mask lists of key block j for the q heads h of K/V head kvh, in
// head order.  Number of entries (before skipping unusable ones).
__device__ __forceinline__ int32_t column_len(const BwdArgs& a, int32_t b, int32_t kvh, int32_t j) {
  const int32_t rep = a.H / a.H_kv;
  int32_t n = 0;
  for (int h = kvh * rep; h < (kvh + 1) * rep; ++h) {
    int32_t e0, e1;
    col_range(a, (int64_t)b * a.mbs + (int64_t)h * a.mhs, j, e0, e1);
    n += e1 - e0;
  }
  return n;
}

// Entries per dK/dV work item: the entries of all columns spread over the
// resident workgroups, at least a.chunk and at most 64 (an item's list is held
// in VGPR lanes).  Columns longer than that are split in chunks, whose fp32
// partials are added atomically; shorter ones are one item each.  The same
// value in every wave (a sum over the heads' mask groups).
__device__ __forceinline__ int32_t chunk_entries(const BwdArgs& a, int lane) {
  int64_t tot = 0;
  for (int64_t x = lane; x < (int64_t)a.B * a.H; x += 64) {
    const int64_t g = (x / a.H) * a.mbs + (x % a.H) * a.mhs;
    int64_t e0 = a.col_ptr[g * a.nb], e1 = a.col_ptr[g * a.nb + a.nb];
    e0 = max((int64_t)0, min(e0, a.row_capacity));
    e1 = max(e0, min(e1, a.row_capacity));
    tot += e1 - e0;
  }
  for (int m = 32; m >= 1; m >>= 1) {
    const int lo = __shfl_xor((int)(uint32_t)tot, m), hi = __shfl_xor((int)(tot >> 32), m);
    tot += ((int64_t)hi << 32) | (uint32_t)lo;
  }
  const int64_t per = (tot + a.slots - 1) / a.slots;
  return (int32_t)max((int64_t)a.chunk, min(per, (int64_t)64));
}

// One wave per column: pre[c + 1] = number of work items (chunks) of column c,
// pre[cols + 1] = entries per chunk; a column split in several chunks gets its
// fp32 partial rows zeroed.
template <int D, int BLK>
__global__ __launch_bounds__(256) void dkdv_plan_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t cols = (int64_t)a.B * a.H_kv * a.nb;
  if (c >= cols) return;
  const int32_t bk = (int32_t)(c / a.nb), j = (int32_t)(c % a.nb);
  const int32_t len = column_len(a, bk / a.H_kv, bk % a.H_kv, j);
  const int32_t L = chunk_entries(a, lane);
  const int32_t chunks = max(1, (len + L - 1) / L);
  if (lane == 0) a.pre[c + 1] = chunks;
  if (c == 0 && lane == 0) a.pre[cols + 1] = L;
  if (chunks > 1) {
    const int64_t plane = (int64_t)a.B * a.H_kv * a.N * D;
    float* r0 = a.acc + ((int64_t)bk * a.N + (int64_t)j * BLK) * D;
    for (int x = lane; x < BLK * D / 4; x += 64) {
      *(sa::f32x4*)(r0 + 4 * x) = sa::f32x4{0.f, 0.f, 0.f, 0.f};
      *(sa::f32x4*)(r0 + plane + 4 * x) = sa::f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// Split columns: fp32 partial sums -> bf16 dk (scaled), dv; kConvWaves waves
// per column, each converting 512 consecutive floats of dK and of dV (8 per
// lane, lanes along the row), so that all of the partials are in flight at once.
template <int D, int BLK>
constexpr int kConvWaves = BLK * D / 512;

template <int D, int BLK>
__global__ __launch_bounds__(256) void dkdv_convert_kernel(BwdArgs a) {
  constexpr int WPC = kConvWaves<D, BLK>;
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t cols = (int64_t)a.B * a.H_kv * a.nb;
  const int64_t c = wv / WPC;
  if (c >= cols || a.pre[c + 1] - a.pre[c] <= 1) return;
  const int32_t bk = (int32_t)(c / a.nb), j = (int32_t)(c % a.nb);
  const int32_t b = bk / a.H_kv, kvh = bk % a.H_kv;
  const int64_t plane = (int64_t)a.B * a.H_kv * a.N * D;
  const int x = (int)(wv % WPC) * 64 + lane;  // 8-float group of the column
  const int r = x / (D / 8), c8 = x % (D / 8);
  const float* pk = a.acc + ((int64_t)bk * a.N + (int64_t)j * BLK + r) * D + 8 * c8;
  const float* pv = pk + plane;
  const sa::f32x4 k0 = *(const sa::f32x4*)pk, k1 = *(const sa::f32x4*)(pk + 4);
  const sa::f32x4 v0 = *(const sa::f32x4*)pv, v1 = *(const sa::f32x4*)(pv + 4);
  const int64_t key = (int64_t)j * BLK + r;
  *(sa::u32x4*)((uint16_t*)a.dk + b * a.st[TDK][0] + kvh * a.st[TDK][1] + key * a.st[TDK][2] + 8 * c8) =
      sa::u32x4{sa::pack_bf16x2(k0[0] * a.scale, k0[1] * a.scale), sa::pack_bf16x2(k0[2] * a.scale, k0[3] * a.scale),
                sa::pack_bf16x2(k1[0] * a.scale, k1[1] * a.scale), sa::pack_bf16x2(k1[2] * a.scale, k1[3] * a.scale)};
  *(sa::u32x4*)((uint16_t*)a.dv + b * a.st[TDV][0] + kvh * a.st[TDV][1] + key * a.st[TDV][2] + 8 * c8) =
      sa::u32x4{sa::pack_bf16x2(v0[0], v0[1]), sa::pack_bf16x2(v0[2], v0[3]), sa::pack_bf16x2(v1[0], v1[1]),
                sa::pack_bf16x2(v1[2], v1[3])};
}

// dk, dv: persistent workgroups (BLK/32 waves, one per 32 keys of the key
// block) take work items = chunks of columns: entries [chunk * C, chunk * C +
// C) of the column's list (C <= 64), so that a key block listed by many query
// blocks (a global block) is shared by several workgroups.  A column with
// one chunk writes its bf16 rows directly; the chunks of a split column add
// their fp32 partials into `acc` (converted afterwards).
//
// The item's query blocks (and their q heads) are held in VGPR lanes; their
// 64-row tiles of Q and dO, with the rows' {lse log2(e), D} pairs, are copied
// global -> LDS by direct loads into a ring of S slots (tile n + S - 1 in
// flight while tile n is used; with one slot the next tile is copied once
// every wave has read the current one).  Wave 0 copies the tile's row
// statistics, which every wave reads after the ring barrier.
//
// The key block's K rows are the B operand of S = Q K^T and stay in registers.
// Its V rows, the B operand of dP = dO V^T, stay in registers too (VL false),
// or (VL true: d = 128, where keeping both takes more than 256 registers, one
// wave per SIMD) are copied once per item into LDS and read back at every use,
// next to a one-slot Q / dO ring: 65 KiB of LDS at block 128, at most 256
// registers, two waves per SIMD.
template <int D, int BLK, int S, bool VL>
__global__ __launch_bounds__(2 * BLK) __attribute__((amdgpu_waves_per_eu(VL ? 2 : 1)))
void bsa_bwd_dkdv_bf16(BwdArgs a) {
  using L = TileLds<D>;
  constexpr int NW = BLK / 32, NU = D / 16, NT = D / 32, SUBS = BLK / 64;
  using M = TileDma<D, NW>;
  constexpr int SLOT = 2 * M::TB + 1024;  // Q tile, dO tile, the rows' statistics
  constexpr int CP = 2 * M::JN;           // tile copies per wave per tile (wave 0: + 1)
  static_assert(S == 2 || S == 3 || (S == 1 && VL), "ring slots");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = sa::uniform(tid >> 6), hl = lane >> 5;
  const int kg = w;  // key group (32 keys) of this wave
  const int32_t rep = a.H / a.H_kv;
  const int64_t cols = (int64_t)a.B * a.H_kv * a.nb;
  const int32_t items = a.pre[cols];
  const int32_t chunkL = sa::uniform(a.pre[cols + 1]);  // entries per chunk, 16 .. 64
  // Items [0, extra) are the second and later chunks of split columns (the
  // long ones, started first); item extra + c is the first chunk of column c.
  const int32_t extra = items - (int32_t)cols;
  const uint32_t ring = sa::lds_addr(smem);
  const uint32_t vblk = ring + S * SLOT;  // V rows of the key block (VL)
  const uint32_t soff = 16u * (uint32_t)(lane & 31);  // statistics: 2 rows per lane, lanes 32.. repeat
  int aoff[NU], troff[NT][2];
#pragma unroll
  for (int u = 0; u < NU; ++u) aoff[u] = L::a_off(u, lane);
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) troff[dt][0] = L::tr_off(dt, 0, lane), troff[dt][1] = L::tr_off(dt, 1, lane);
  bool first = true;
  for (int32_t item = blockIdx.x; item < items; item += gridDim.x) {
    int64_t c;
    int32_t chunk;
    if (item >= extra) {
      // first chunks in (j, bk) order: consecutive items take the same key
      // block of different heads, so (B * H_kv a multiple of 8) every key
      // block of one head runs on the same XCD, like its query blocks
      const int32_t x = item - extra, bhk = a.B * a.H_kv;
      c = (int64_t)(x % bhk) * a.nb + x / bhk;
      chunk = 0;
    } else {
      // pre[c] - c counts the extra chunks of the columns before c: the item's
      // column is the last c with pre[c] - c <= item
      int64_t lo = 0, hi = cols;
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (a.pre[mid] - mid <= item)
          lo = mid;
        else
          hi = mid;
      }
      c = lo;
      chunk = 1 + item - (int32_t)(a.pre[c] - c);
    }
    c = sa::uniform((int32_t)c);
    chunk = sa::uniform(chunk);
    const int split = sa::uniform((int)(a.pre[c + 1] - a.pre[c] > 1));
    const int32_t bk = (int32_t)(c / a.nb), j = (int32_t)(c % a.nb);
    const int32_t b = bk / a.H_kv, kvh = bk % a.H_kv;
    const int32_t f0 = chunk * chunkL;  // first flat entry of this item
    const int koff = 32 * kg + (lane & 31);       // this lane's key inside the block
    const int64_t sk = (int64_t)j * BLK + koff;   // ... and in the sequence (C column)
    const uint16_t* K = (const uint16_t*)a.k + b * a.st[TK][0] + kvh * a.st[TK][1];
    const uint16_t* V = (const uint16_t*)a.v + b * a.st[TV][0] + kvh * a.st[TV][1];
    sa::u32x4 kb_[NU], vb_[VL ? 1 : NU];  // B operands: column = key, k = d
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      kb_[u] = *(const sa::u32x4*)(K + sk * a.st[TK][2] + 16 * u + 8 * hl);
      if constexpr (!VL) vb_[u] = *(const sa::u32x4*)(V + sk * a.st[TV][2] + 16 * u + 8 * hl);
    }
    // the item's entries: flat entry f0 + x (over the heads in order) in lane x
    int32_t lq = -1, lh = 0, total = 0;
    for (int h = kvh * rep; h < (kvh + 1) * rep; ++h) {
      int32_t e0, e1;
      col_range(a, (int64_t)b * a.mbs + (int64_t)h * a.mhs, j, e0, e1);
      const int32_t x = f0 + lane - total;
      if (lane < chunkL && x >= 0 && x < e1 - e0) {
        const int32_t qb = a.row_idx[e0 + x];
        lq = ((uint32_t)qb < (uint32_t)a.nb && !(a.causal && qb < j)) ? qb : -1;
        lh = h;
      }
      total += e1 - e0;
    }
    const int cnt = sa::uniform(max(0, min(chunkL, total - f0)));
    // the loads above complete here, before any copy is in flight (stores of
    // the previous item included)
#pragma unroll
    for (int u = 0; u < NU; ++u) sa::keep(kb_[u]);
    if constexpr (!VL)
#pragma unroll
      for (int u = 0; u < NU; ++u) sa::keep(vb_[u]);
    sa::keep(lq), sa::keep(lh), sa::keep(split);
    sa::vm_wait<0>();
    if (!first) ring_barrier();  // every wave is done with the ring (and the V rows)
    first = false;

    sa::f32x16 dk[NT], dv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) dk[t] = sa::f32x16{}, dv[t] = sa::f32x16{};
    const int T = cnt * SUBS;
    auto issue = [&](int m) {
      // without grouped query heads every entry's head is the K/V head
      const int32_t qb = sa::readlane(lq, m / SUBS), h = rep == 1 ? kvh : sa::readlane(lh, m / SUBS);
      const int64_t r0 = (int64_t)(qb < 0 ? j : qb) * BLK + 64 * (m % SUBS);
      const uint16_t* Q = (const uint16_t*)a.q + b * a.st[TQ][0] + h * a.st[TQ][1];
      const uint16_t* G = (const uint16_t*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1];
      const float* st = (const float*)(a.stat + ((int64_t)b * a.H + h) * a.N + r0);
      const uint32_t dst = ring + (m % S) * SLOT;
      // the per-lane source offsets are recomputed here (a few VALU
      // instructions) from a fresh lane id: hoisted out of the tile loop they
      // were spilled, and every copy waited for their reload
      const int ln = sa::fresh_lane();
      M::copy(Q + r0 * a.st[TQ][2], a.st[TQ][2], M::lane_off(w, ln, a.st[TQ][2]), dst, w);
      M::copy(G + r0 * a.st[TDO][2], a.st[TDO][2], M::lane_off(w, ln, a.st[TDO][2]), dst + M::TB, w);
      if (w == 0) sa::dma16(st, 16u * (uint32_t)(ln & 31), dst + 2 * M::TB);
    };
    if constexpr (VL) {
      // the key block's V rows, 64-row tiles one after the other
#pragma unroll
      for (int sub = 0; sub < SUBS; ++sub)
        M::copy(V + ((int64_t)j * BLK + 64 * sub) * a.st[TV][2], a.st[TV][2], M::lane_off(w, lane, a.st[TV][2]),
                vblk + sub * M::TB, w);
    }
    if (T > 0) issue(0);
    if (S > 2 && T > 1) issue(1);
    for (int n = 0; n < T; ++n) {
      if constexpr (S == 1) {
        sa::vm_wait<0>();
        ring_barrier();
      } else {
        if (w == 0)
          wait_units<CP + 1>(S > 2 && n + 1 < T);
        else
          wait_units<CP>(S > 2 && n + 1 < T);
        ring_barrier();
        if (n + S - 1 < T) issue(n + S - 1);
      }
      const int32_t qb = sa::readlane(lq, n / SUBS);
      if (qb >= 0) {
        const uint8_t* qs = smem + (n % S) * SLOT;
        const uint8_t* gs = qs + M::TB;
        const float* sts = (const float*)(gs + M::TB);
        const int qsub = 64 * (n % SUBS);
        const bool diag = a.causal && qb == j;
        // one 32-query half; the causal triangle applies when diag
        auto half = [&](int qt) {
          // V rows of this wave's keys, read again for every half (the opaque
          // base keeps the compiler from holding them in registers)
          uint32_t vrows = vblk + (uint32_t)(32 * kg / 64) * M::TB;
          asm volatile("" : "+s"(vrows));
          // S and dP [32 queries x 32 keys]: MFMA m = 2u takes the Q rows,
          // m = 2u + 1 the dO rows (and, VL, the V rows); their reads are issued
          // LA MFMAs ahead of use (scheduling barriers hold the order; the
          // compiler counts the reads in its waits)
          constexpr int NA = 2 * NU, LA = 2;
          sa::u32x4 qa[NU], ga[NU], va[VL ? NU : 1];
          const uint8_t* qh = qs + 32 * qt * L::ROWB;  // the half's 32 Q rows (dO: M::TB further)
          auto ard = [&](auto m) {
            constexpr int Mi = decltype(m)::value, U = Mi >> 1;
            if constexpr (Mi < NA && (Mi & 1) == 0) qa[U] = L::at_a(qh, aoff[U]);
            if constexpr (Mi < NA && (Mi & 1) == 1) {
              ga[U] = L::at_a(qh + M::TB, aoff[U]);
              if constexpr (VL) va[U] = L::rows_a_lds(vrows, (32 * kg) % 64, U, lane);
            }
          };
          sa::static_for<0, LA>(ard);
          sa::f32x16 s, dp;
          sa::static_for<0, NA>([&](auto m) {
            constexpr int Mi = decltype(m)::value, U = Mi >> 1;
            SA_SCHED_BARRIER();
            if constexpr (Mi & 1) {
              sa::u32x4 vop;
              if constexpr (VL)
                vop = va[U];
              else
                vop = vb_[U];
              dp = Mi == 1 ? sa::mfma32_z(ga[U], vop) : sa::mfma32(ga[U], vop, dp);
            } else {
              s = Mi == 0 ? sa::mfma32_z(qa[U], kb_[U]) : sa::mfma32(qa[U], kb_[U], s);
            }
            ard(std::integral_constant<int, Mi + LA>{});
          });
          SA_SCHED_BARRIER();
          // transposed A operands of dV^T += dO^T P and dK^T += Q^T dS, j =
          // st NT + dt; the first in flight during the VALU work below
          constexpr int NC = 2 * NT;
          sa::u32x4 gt[NC], qtr[NC];
          auto crd = [&](auto jj) {
            constexpr int J = decltype(jj)::value;
            if constexpr (J < NC) {
              const uint8_t* qb16 = qh + 16 * (J / NT) * L::ROWB;
              gt[J] = L::at_tr(qb16 + M::TB, troff[J % NT][0], troff[J % NT][1]);
              qtr[J] = L::at_tr(qb16, troff[J % NT][0], troff[J % NT][1]);
            }
          };
          crd(std::integral_constant<int, 0>{});
          float p[16], ds[16];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int q4 = 32 * qt + 8 * r4 + 4 * hl;  // 4 consecutive query rows of the tile
            const sa::f32x4 x0 = *(const sa::f32x4*)(sts + 2 * q4);  // {l, D} of rows q4, q4 + 1
            const sa::f32x4 x1 = *(const sa::f32x4*)(sts + 2 * q4 + 4);
            const float lv[4] = {x0[0], x0[2], x1[0], x1[2]}, dv4[4] = {x0[1], x0[3], x1[1], x1[3]};
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
              const int r = 4 * r4 + cc;
              p[r] = sa::fast_exp2(__builtin_fmaf(s[r], a.c2, -lv[cc]));
              ds[r] = p[r] * (dp[r] - dv4[cc]);
            }
          }
          if (diag) {
            // keys after the query (diagonal tile only: a wave-uniform branch,
            // kept as one by the volatile asm, so other tiles skip the selects)
            asm volatile("" ::: "memory");
            // this lane's key less its row offset 4 hl, from a fresh lane id
            // (no register is held across the tile loop for it)
            const int fl = sa::fresh_lane();
            const int kd = 32 * kg + (fl & 31) - 4 * (fl >> 5) - qsub - 32 * qt;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kd > 8 * (r >> 2) + (r & 3)) p[r] = 0.f, ds[r] = 0.f;
          }
          // dV^T += dO^T P,  dK^T += Q^T dS   ([d x queries] x [queries x keys])
          const sa::u32x4 pb[2] = {pack8(p), pack8(p + 8)}, sb[2] = {pack8(ds), pack8(ds + 8)};
          crd(std::integral_constant<int, 1>{});  // two ahead from here on
          sa::static_for<0, NC>([&](auto jj) {
            constexpr int J = decltype(jj)::value;
            SA_SCHED_BARRIER();
            dv[J % NT] = sa::mfma32(gt[J], pb[J / NT], dv[J % NT]);
            dk[J % NT] = sa::mfma32(qtr[J], sb[J / NT], dk[J % NT]);
            crd(std::integral_constant<int, J + 2>{});
          });
          SA_SCHED_BARRIER();
        };
        bwd_tile(half);
      }
      if constexpr (S == 1) {
        if (n + 1 < T) {
          // every wave has read tile n (its LDS reads returned): refill the slot
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          ring_barrier();
          issue(n + 1);
        }
      }
    }
// C rows of tile dt are d = 32 dt + 8(r/4) + 4(l/32) + r%4 of this lane's key
    if (!split) {
      uint16_t* DK = (uint16_t*)a.dk + b * a.st[TDK][0] + kvh * a.st[TDK][1] + sk * a.st[TDK][2];
      uint16_t* DV = (uint16_t*)a.dv + b * a.st[TDV][0] + kvh * a.st[TDV][1] + sk * a.st[TDV][2];
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const sa::f32x16& x = dk[dt];
          const sa::f32x16& y = dv[dt];
          const int r = 4 * r4;
          *(sa::u32x2*)(DK + 32 * dt + 8 * r4 + 4 * hl) = sa::u32x2{
              sa::pack_bf16x2(x[r] * a.scale, x[r + 1] * a.scale), sa::pack_bf16x2(x[r + 2] * a.scale, x[r + 3] * a.scale)};
          *(sa::u32x2*)(DV + 32 * dt + 8 * r4 + 4 * hl) =
              sa::u32x2{sa::pack_bf16x2(y[r], y[r + 1]), sa::pack_bf16x2(y[r + 2], y[r + 3])};
        }
    } else {
      // A chunk of a split column adds its fp32 partials into the workspace.
      // They go through LDS (free once the tile loop is done), dK then dV, so
      // that each atomic instruction covers 64 consecutive floats of one key
      // row (two cache lines) rather than one float in each of 32 rows; the
      // 16-byte chunks of a staged row are XOR-swizzled by the key's low four
      // bits, which keeps the writes of 16 keys at one chunk conflict-free.
      static_assert(S * SLOT + (VL ? BLK * 2 * D : 0) >= BLK * D * 4, "staging area");
      const int64_t plane = (int64_t)a.B * a.H_kv * a.N * D;
      float* const pk = a.acc + ((int64_t)bk * a.N + (int64_t)j * BLK) * D;
      float* const stage = (float*)smem;
      const int kl = 32 * kg + (lane & 31);  // this lane's key in the block
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      ring_barrier();  // every wave is done with the ring and the V rows
#pragma unroll
      for (int mtx = 0; mtx < 2; ++mtx) {
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const sa::f32x16& x = mtx == 0 ? dk[dt] : dv[dt];
            const int c = 8 * dt + 2 * r4 + hl;  // 16-byte chunk of d 32 dt + 8 r4 + 4 hl .. + 3
            *(sa::f32x4*)(stage + kl * D + 4 * (c ^ (kl & 15))) =
                sa::f32x4{x[4 * r4], x[4 * r4 + 1], x[4 * r4 + 2], x[4 * r4 + 3]};
          }
        __syncthreads();
        float* const dst = pk + (mtx == 0 ? 0 : plane);
#pragma unroll 4
        for (int i = 0; i < D / 2; ++i) {
          const int e = tid + i * 2 * BLK;  // element (key e / D, d e % D) of the block
          const int k = e / D, d = e % D;
          atomicAdd(dst + e, stage[k * D + 4 * ((d >> 2) ^ (k & 15)) + (d & 3)]);
        }
        __syncthreads();  // the staging area is reused for dV
      }
    }
  }
}

// --------------------------------------------------------------- offsets ---
// dq: one thread per query; keys t - delta.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void off_bwd_dq(BwdArgs a) {
  typedef typename Elem<BF16>::T T;
  const int tiles = (a.N + 255) / 256;
  const int32_t bh = blockIdx.x / tiles;
  const int64_t t = (int64_t)(blockIdx.x % tiles) * 256 + threadIdx.x;
  if (t >= a.N) return;
  const int32_t b = bh / a.H, h = bh % a.H, kvh = h / (a.H / a.H_kv);
  const T* K = (const T*)a.k + b * a.st[TK][0] + kvh * a.st[TK][1];
  const T* V = (const T*)a.v + b * a.st[TV][0] + kvh * a.st[TV][1];
  float qv[D], gv[D], acc[D];
  load_f<D, BF16>((const T*)a.q + b * a.st[TQ][0] + h * a.st[TQ][1] + t * a.st[TQ][2], qv);
  load_f<D, BF16>((const T*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1] + t * a.st[TDO][2], gv);
#pragma unroll
  for (int x = 0; x < D; ++x) acc[x] = 0.f;
  const int64_t row = ((int64_t)b * a.H + h) * a.N + t;
  const float l2 = lse2_of(a.lse[row]), dd = a.delta[row];
  for (int n = 0; n < a.noff && a.offs[n] <= t; ++n) {
    const int64_t src = t - a.offs[n];
    float kf[D], vf[D];
    load_f<D, BF16>(K + src * a.st[TK][2], kf);
    load_f<D, BF16>(V + src * a.st[TV][2], vf);
    float dot = 0.f, dp = 0.f;
#pragma unroll
    for (int x = 0; x < D; ++x) dot = fmaf(qv[x], kf[x], dot), dp = fmaf(gv[x], vf[x], dp);
    const float ds = exp2f(dot * a.c2 - l2) * (dp - dd);
#pragma unroll
    for (int x = 0; x < D; ++x) acc[x] = fmaf(ds, kf[x], acc[x]);
  }
#pragma unroll
  for (int x = 0; x < D; ++x) acc[x] *= a.scale;
  store_f<D, BF16>((T*)a.dq + b * a.st[TDQ][0] + h * a.st[TDQ][1] + t * a.st[TDQ][2], acc);
}

// dk, dv: one thread per key s of a K/V head; queries s + delta of every q head
// of the group.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void off_bwd_dkdv(BwdArgs a) {
  typedef typename Elem<BF16>::T T;
  const int tiles = (a.N + 255) / 256;
  const int32_t bk = blockIdx.x / tiles;
  const int64_t s = (int64_t)(blockIdx.x % tiles) * 256 + threadIdx.x;
  if (s >= a.N) return;
  const int32_t b = bk / a.H_kv, kvh = bk % a.H_kv, rep = a.H / a.H_kv;
  float kv[D], vv[D], dk[D], dv[D];
  load_f<D, BF16>((const T*)a.k + b * a.st[TK][0] + kvh * a.st[TK][1] + s * a.st[TK][2], kv);
  load_f<D, BF16>((const T*)a.v + b * a.st[TV][0] + kvh * a.st[TV][1] + s * a.st[TV][2], vv);
#pragma unroll
  for (int x = 0; x < D; ++x) dk[x] = dv[x] = 0.f;
  for (int h = kvh * rep; h < (kvh + 1) * rep; ++h) {
    const T* Q = (const T*)a.q + b * a.st[TQ][0] + h * a.st[TQ][1];
    const T* G = (const T*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1];
    const int64_t rowb = ((int64_t)b * a.H + h) * a.N;
    for (int n = 0; n < a.noff && s + a.offs[n] < a.N; ++n) {
      const int64_t t = s + a.offs[n];
      float qf[D], gf[D];
      load_f<D, BF16>(Q + t * a.st[TQ][2], qf);
      load_f<D, BF16>(G + t * a.st[TDO][2], gf);
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) dot = fmaf(qf[x], kv[x], dot), dp = fmaf(gf[x], vv[x], dp);
      const float p = exp2f(dot * a.c2 - lse2_of(a.lse[rowb + t]));
      const float ds = p * (dp - a.delta[rowb + t]);
#pragma unroll
      for (int x = 0; x < D; ++x) dk[x] = fmaf(ds, qf[x], dk[x]), dv[x] = fmaf(p, gf[x], dv[x]);
    }
  }
#pragma unroll
  for (int x = 0; x < D; ++x) dk[x] *= a.scale;
  store_f<D, BF16>((T*)a.dk + b * a.st[TDK][0] + kvh * a.st[TDK][1] + s * a.st[TDK][2], dk);
  store_f<D, BF16>((T*)a.dv + b * a.st[TDV][0] + kvh * a.st[TDV][1] + s * a.st[TDV][2], dv);
}

// bf16 offset gradients: four lanes per row (lane 4 r + j holds 16-byte chunks
// 4 c + j of its row), 16 rows per wave, so the 4 lanes reading one row are
// adjacent (one 64-byte segment per group of 4 lanes); dot products are
// reduced over the quad with DPP.  Distances are taken OB at a time (loads
// first, then the arithmetic).
constexpr int OB = 4;

__device__ __forceinline__ void unpack8(const sa::u32x4& w, float* f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) f[2 * j] = sa::bf16_lo(w[j]), f[2 * j + 1] = sa::bf16_hi(w[j]);
}

template <int D>
__global__ __launch_bounds__(256) void off_bwd_dq_bf16(BwdArgs a) {
  constexpr int NC = D / 32;
  const int tiles = (a.N + 63) / 64;
  const int32_t bh = blockIdx.x / tiles;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, rq = lane >> 2, j = lane & 3;
  const int64_t t = (int64_t)(blockIdx.x % tiles) * 64 + 16 * w + rq;
  const bool live = t < a.N;
  const int64_t tq = live ? t : a.N - 1;
  const int32_t b = bh / a.H, h = bh % a.H, kvh = h / (a.H / a.H_kv);
  const uint16_t* K = (const uint16_t*)a.k + b * a.st[TK][0] + kvh * a.st[TK][1];
  const uint16_t* V = (const uint16_t*)a.v + b * a.st[TV][0] + kvh * a.st[TV][1];
  const uint16_t* Q = (const uint16_t*)a.q + b * a.st[TQ][0] + h * a.st[TQ][1] + tq * a.st[TQ][2];
  const uint16_t* G = (const uint16_t*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1] + tq * a.st[TDO][2];
  sa::u32x4 qv[NC], gv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qv[c] = *(const sa::u32x4*)(Q + 8 * (4 * c + j)), gv[c] = *(const sa::u32x4*)(G + 8 * (4 * c + j));
  float acc[8 * NC];
#pragma unroll
  for (int x = 0; x < 8 * NC; ++x) acc[x] = 0.f;
  const int64_t row = ((int64_t)b * a.H + h) * a.N + tq;
  const float l2 = lse2_of(a.lse[row]), dd = a.delta[row];
  for (int n0 = 0; n0 < a.noff; n0 += OB) {
    sa::u32x4 kr[OB][NC], vr[OB][NC];
    bool ok[OB];
#pragma unroll
    for (int u = 0; u < OB; ++u) {
      const int n = min(n0 + u, a.noff - 1);
      ok[u] = n0 + u < a.noff && tq >= a.offs[n];
      const int64_t src = max(tq - a.offs[n], (int64_t)0);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        kr[u][c] = *(const sa::u32x4*)(K + src * a.st[TK][2] + 8 * (4 * c + j));
        vr[u][c] = *(const sa::u32x4*)(V + src * a.st[TV][2] + 8 * (4 * c + j));
      }
    }
#pragma unroll
    for (int u = 0; u < OB; ++u) {
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int x = 0; x < 4; ++x) dot = sa::dot2_bf16(qv[c][x], kr[u][c][x], dot), dp = sa::dot2_bf16(gv[c][x], vr[u][c][x], dp);
      dot = sa::quad_sum(dot);
      dp = sa::quad_sum(dp);
      const float ds = ok[u] ? exp2f(dot * a.c2 - l2) * (dp - dd) : 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float kf[8];
        unpack8(kr[u][c], kf);
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[8 * c + x] = fmaf(ds, kf[x], acc[8 * c + x]);
      }
    }
  }
  if (!live) return;
  uint16_t* DQ = (uint16_t*)a.dq + b * a.st[TDQ][0] + h * a.st[TDQ][1] + t * a.st[TDQ][2];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    sa::u32x4 wv;
#pragma unroll
    for (int x = 0; x < 4; ++x) wv[x] = sa::pack_bf16x2(acc[8 * c + 2 * x] * a.scale, acc[8 * c + 2 * x + 1] * a.scale);
    *(sa::u32x4*)(DQ + 8 * (4 * c + j)) = wv;
  }
}

template <int D>
__global__ __launch_bounds__(256) void off_bwd_dkdv_bf16(BwdArgs a) {
  constexpr int NC = D / 32;
  const int tiles = (a.N + 63) / 64;
  const int32_t bk = blockIdx.x / tiles;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, rk = lane >> 2, j = lane & 3;
  const int64_t s = (int64_t)(blockIdx.x % tiles) * 64 + 16 * w + rk;
  const bool live = s < a.N;
  const int64_t sk = live ? s : a.N - 1;
  const int32_t b = bk / a.H_kv, kvh = bk % a.H_kv, rep = a.H / a.H_kv;
  const uint16_t* K = (const uint16_t*)a.k + b * a.st[TK][0] + kvh * a.st[TK][1] + sk * a.st[TK][2];
  const uint16_t* V = (const uint16_t*)a.v + b * a.st[TV][0] + kvh * a.st[TV][1] + sk * a.st[TV][2];
  sa::u32x4 kv[NC], vv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) kv[c] = *(const sa::u32x4*)(K + 8 * (4 * c + j)), vv[c] = *(const sa::u32x4*)(V + 8 * (4 * c + j));
  float dk[8 * NC], dv[8 * NC];
#pragma unroll
  for (int x = 0; x < 8 * NC; ++x) dk[x] = dv[x] = 0.f;
  for (int h = kvh * rep; h < (kvh + 1) * rep; ++h) {
    const uint16_t* Q = (const uint16_t*)a.q + b * a.st[TQ][0] + h * a.st[TQ][1];
    const uint16_t* G = (const uint16_t*)a.dout + b * a.st[TDO][0] + h * a.st[TDO][1];
    const int64_t rowb = ((int64_t)b * a.H + h) * a.N;
    for (int n0 = 0; n0 < a.noff; n0 += OB) {
      sa::u32x4 qr[OB][NC], gr[OB][NC];
      float l2[OB], dd[OB];
      bool ok[OB];
#pragma unroll
      for (int u = 0; u < OB; ++u) {
        const int n = min(n0 + u, a.noff - 1);
        const int64_t t = sk + a.offs[n];
        ok[u] = n0 + u < a.noff && t < a.N;
        const int64_t tt = min(t, (int64_t)a.N - 1);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          qr[u][c] = *(const sa::u32x4*)(Q + tt * a.st[TQ][2] + 8 * (4 * c + j));
          gr[u][c] = *(const sa::u32x4*)(G + tt * a.st[TDO][2] + 8 * (4 * c + j));
        }
        l2[u] = lse2_of(a.lse[rowb + tt]);
        dd[u] = a.delta[rowb + tt];
      }
#pragma unroll
      for (int u = 0; u < OB; ++u) {
        float dot = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int x = 0; x < 4; ++x) dot = sa::dot2_bf16(qr[u][c][x], kv[c][x], dot), dp = sa::dot2_bf16(gr[u][c][x], vv[c][x], dp);
        dot = sa::quad_sum(dot);
        dp = sa::quad_sum(dp);
        const float p = ok[u] ? exp2f(dot * a.c2 - l2[u]) : 0.f;
        const float ds = p * (dp - dd[u]);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float qf[8], gf[8];
          unpack8(qr[u][c], qf);
          unpack8(gr[u][c], gf);
#pragma unroll
          for (int x = 0; x < 8; ++x) dk[8 * c + x] = fmaf(ds, qf[x], dk[8 * c + x]), dv[8 * c + x] = fmaf(p, gf[x], dv[8 * c + x]);
        }
      }
    }
  }
  if (!live) return;
  uint16_t* DK = (uint16_t*)a.dk + b * a.st[TDK][0] + kvh * a.st[TDK][1] + s * a.st[TDK][2];
  uint16_t* DV = (uint16_t*)a.dv + b * a.st[TDV][0] + kvh * a.st[TDV][1] + s * a.st[TDV][2];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    sa::u32x4 w1, w2;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      w1[x] = sa::pack_bf16x2(dk[8 * c + 2 * x] * a.scale, dk[8 * c + 2 * x + 1] * a.scale);
      w2[x] = sa::pack_bf16x2(dv[8 * c + 2 * x], dv[8 * c + 2 * x + 1]);
    }
    *(sa::u32x4*)(DK + 8 * (4 * c + j)) = w1;
    *(sa::u32x4*)(DV + 8 * (4 * c + j)) = w2;
  }
}

// ------------------------------------------------------------------ host ---
template <typename F>
sa_status launch(F kern, const BwdArgs& a, int64_t blocks, int threads, int lds, hipStream_t stream,
                 const char* what) {
  if (blocks <= 0) return SA_OK;
  if (blocks > 0x7fffffffll) return SA_ERR_UNSUPPORTED;
  const sa_status ls = allow_lds((const void*)kern, lds);
  if (ls != SA_OK) return ls;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(threads), lds, stream, a);
  return sa_host::check_launch(what);
}

// Shared argument checks of both backward entry points; fills a.
sa_status common_args(BwdArgs& a, int32_t dtype, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, float* delta, int32_t B,
                      int32_t H, int32_t H_kv, int32_t N, int32_t d, const int64_t* strides, float scale) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return SA_ERR_NULL;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_INVALID;
  if (B < 1 || H < 1 || H_kv < 1 || N < 1 || d < 1 || H % H_kv != 0) return SA_ERR_INVALID;
  if (!isfinite(scale)) return SA_ERR_INVALID;
  if (d != 64 && d != 128) return SA_ERR_UNSUPPORTED;
  const void* ptrs[8] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!sa_host::aligned16(p)) return SA_ERR_INVALID;
  const int32_t heads[8] = {H, H_kv, H_kv, H, H, H, H_kv, H_kv};
  const int align = dtype == SA_BF16 ? 8 : 4;
  for (int t = 0; t < 8; ++t) {
    int64_t sb, sh, ss;
    if (!strides) {
      ss = d, sh = (int64_t)N * d, sb = (int64_t)heads[t] * N * d;
    } else {
      sb = strides[3 * t], sh = strides[3 * t + 1], ss = strides[3 * t + 2];
    }
    if (ss < d || sh < 0 || sb < 0 || ss % align || sh % align || sb % align) return SA_ERR_INVALID;
    a.st[t][0] = sb, a.st[t][1] = sh, a.st[t][2] = ss;
  }
  a.q = q, a.k = k, a.v = v, a.o = o, a.dout = dout, a.dq = dq, a.dk = dk, a.dv = dv;
  a.lse = lse, a.delta = delta;
  a.B = B, a.H = H, a.H_kv = H_kv, a.N = N;
  a.scale = scale, a.c2 = scale * sa::kLog2e;
  return SA_OK;
}

sa_status launch_delta(const BwdArgs& a, int32_t dtype, int32_t d, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const int64_t blocks = (rows * (d / 8) + 255) / 256;
  if (dtype == SA_BF16)
    return d == 64 ? launch(delta_kernel<64, true>, a, blocks, 256, 0, stream, "delta_kernel")
                   : launch(delta_kernel<128, true>, a, blocks, 256, 0, stream, "delta_kernel");
  return d == 64 ? launch(delta_kernel<64, false>, a, blocks, 256, 0, stream, "delta_kernel")
                 : launch(delta_kernel<128, false>, a, blocks, 256, 0, stream, "delta_kernel");
}

// Least CSR entries per dK/dV work item (chunks grow up to 64 entries when
// the columns' entries outnumber the resident workgroups).
constexpr int kChunkEntries = 16;

// Workgroups of `kern` resident on the current device at once (cached per
// device and kernel).  The value only sizes the dK/dV work items, so a failed
// query falls back to one workgroup per CU of a 256-CU device (and its error
// is cleared here rather than left for the caller's next HIP call).
int64_t resident_workgroups(const void* kern, int threads, int lds) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int64_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kern);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  const hipError_t e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds);
  const hipError_t e2 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e1 != hipSuccess || e2 != hipSuccess) (void)hipGetLastError();
  if (e1 != hipSuccess || per_cu < 1) per_cu = 1;
  if (e2 != hipSuccess || cus < 1) cus = 256;
  return cache[key] = (int64_t)per_cu * cus;
}


template <int D, int BLK>
sa_status launch_bsa_bwd(const BwdArgs& a, bool bf16, hipStream_t stream) {
  const int64_t nq = (int64_t)a.B * a.H * a.nb, nk = (int64_t)a.B * a.H_kv * a.nb;
  sa_status st;
  if (bf16) {
    // d = 128: the dK/dV kernel keeps V in LDS beside a one-slot ring (two
    // waves per SIMD); d = 64: V in registers and a two-slot ring
    constexpr int SQ = 2;
    constexpr bool VL = D == 128;
    constexpr int SK = VL ? 1 : 2;
    constexpr int lds_dq = SQ * 2 * TileDma<D, BLK / 32>::TB;
    constexpr int lds_kv = SK * (2 * TileDma<D, BLK / 32>::TB + 1024) + (VL ? BLK * 2 * D : 0);
    st = launch(bsa_bwd_dq_bf16<D, BLK, SQ>, a, nq, 2 * BLK, lds_dq, stream, "bsa_bwd_dq_bf16");
    if (st != SA_OK) return st;
    const int64_t wblocks = (nk + 3) / 4;
    const sa_status ls = allow_lds((const void*)bsa_bwd_dkdv_bf16<D, BLK, SK, VL>, lds_kv);
    if (ls != SA_OK) return ls;
    BwdArgs ap = a;
    ap.slots = resident_workgroups((const void*)bsa_bwd_dkdv_bf16<D, BLK, SK, VL>, 2 * BLK, lds_kv);
    st = launch(dkdv_plan_kernel<D, BLK>, ap, wblocks, 256, 0, stream, "dkdv_plan_kernel");
    if (st != SA_OK) return st;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, a.pre, nk);
    st = sa_host::check_launch("scan_kernel");
    if (st != SA_OK) return st;
    // persistent workgroups; the item count lives on the device
    st = launch(bsa_bwd_dkdv_bf16<D, BLK, SK, VL>, a, std::min<int64_t>(nk + nk / 2 + 64, 8192), 2 * BLK, lds_kv,
                stream, "bsa_bwd_dkdv_bf16");
    if (st != SA_OK) return st;
    return launch(dkdv_convert_kernel<D, BLK>, a, (nk * kConvWaves<D, BLK> + 3) / 4, 256, 0, stream,
                  "dkdv_convert_kernel");
  }
  st = launch(bsa_bwd_dq_f32<D, BLK>, a, nq, BLK, 0, stream, "bsa_bwd_dq_f32");
  if (st != SA_OK) return st;
  return launch(bsa_bwd_dkdv_f32<D, BLK>, a, nk, BLK, 0, stream, "bsa_bwd_dkdv_f32");
}

// Workspace of sparse_attn_bwd: row statistics fp32 [B*H*N][2] ({lse log2(e),
// D} pairs; D alone in the first half for fp32) | pre int32 [B*H_kv*nb + 2] |
// acc fp32 [2][B*H_kv*N*d], each part 256-byte aligned.
struct WsLayout {
  int64_t stat, pre, acc, total;
};
WsLayout ws_layout(int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, int64_t block) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  WsLayout l;
  l.stat = 0;
  l.pre = up(B * H * N * 8);
  l.acc = l.pre + up((B * H_kv * (N / block) + 2) * 4);
  l.total = l.acc + up(2 * B * H_kv * N * d * 4);
  return l;
}

}  // namespace

extern "C" int64_t sparse_attn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                                                   int32_t block) {
  if (B < 1 || H < 1 || H_kv < 1 || N < 1 || d < 1 || block < 1) return SA_ERR_INVALID;
  return ws_layout(B, H, H_kv, N, d, block).total;
}

extern "C" sa_status sparse_attn_mask_transpose(int32_t num_groups, int32_t num_blocks, const int32_t* row_ptr,
                                                const int32_t* col_idx, int64_t col_capacity, int32_t* col_ptr,
                                                int32_t* row_idx, int64_t row_capacity, hipStream_t stream) {
  if (!row_ptr || !col_idx || !col_ptr || !row_idx) return SA_ERR_NULL;
  if (num_groups < 1 || num_blocks < 1 || num_blocks > SA_MAX_BLOCKS || col_capacity < 0 || row_capacity < 0)
    return SA_ERR_INVALID;
  const int64_t cols = (int64_t)num_groups * num_blocks;
  if (cols >= 0x7fffffffll) return SA_ERR_UNSUPPORTED;
  TrArgs t = {row_ptr, col_idx, col_ptr, row_idx, col_capacity, row_capacity, num_groups, num_blocks};
  const unsigned blocks = (unsigned)((cols + 3) / 4);
  hipLaunchKernelGGL((transpose_kernel<false>), dim3(blocks), dim3(256), 0, stream, t);
  sa_status st = sa_host::check_launch("transpose_kernel<count>");
  if (st != SA_OK) return st;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, col_ptr, cols);
  st = sa_host::check_launch("scan_kernel");
  if (st != SA_OK) return st;
  hipLaunchKernelGGL((transpose_kernel<true>), dim3(blocks), dim3(256), 0, stream, t);
  return sa_host::check_launch("transpose_kernel<fill>");
}

extern "C" sa_status sparse_attn_bwd(int32_t dtype, const void* q, const void* k, const void* v, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                     void* workspace, int64_t workspace_bytes, int32_t B, int32_t H,
                                     int32_t H_kv, int32_t N, int32_t d,
                                     int32_t block, const int64_t* strides, const int32_t* row_ptr,
                                     const int32_t* col_idx, int64_t col_capacity, const int32_t* sched,
                                     const int32_t* col_ptr,
                                     const int32_t* row_idx, int64_t row_capacity, int32_t num_groups,
                                     int64_t mask_batch_stride, int64_t mask_head_stride, int32_t causal,
                                     float scale, hipStream_t stream) {
  BwdArgs a = {};
  if (!row_ptr || !col_idx || !col_ptr || !row_idx || !workspace) return SA_ERR_NULL;
  if (!sa_host::aligned16(workspace) || block < 1) return SA_ERR_INVALID;
  const WsLayout wsl = ws_layout(B > 0 ? B : 1, H > 0 ? H : 1, H_kv > 0 ? H_kv : 1, N > 0 ? N : 1,
                                 d > 0 ? d : 1, block);
  if (workspace_bytes < wsl.total) return SA_ERR_CAPACITY;
  uint8_t* ws = (uint8_t*)workspace;
  sa_status st = common_args(a, dtype, q, k, v, o, lse, dout, dq, dk, dv, (float*)(ws + wsl.stat), B, H, H_kv,
                             N, d, strides, scale);
  if (st != SA_OK) return st;
  a.stat = (sa::f32x2*)(ws + wsl.stat);
  a.pre = (int32_t*)(ws + wsl.pre);
  a.acc = (float*)(ws + wsl.acc);
  a.chunk = kChunkEntries;  // CSR entries per item
  if (block < 1 || causal < 0 || causal > 1 || col_capacity < 0 || row_capacity < 0) return SA_ERR_INVALID;
  if (num_groups < 1 || mask_batch_stride < 0 || mask_head_stride < 0) return SA_ERR_INVALID;
  if ((int64_t)(B - 1) * mask_batch_stride + (int64_t)(H - 1) * mask_head_stride >= num_groups)
    return SA_ERR_INVALID;
  if (N % block != 0) return SA_ERR_INVALID;
  if (block != 64 && block != 128) return SA_ERR_UNSUPPORTED;
  // the bf16 kernels keep the byte offsets of the rows of a 64-row tile in 32 bits
  if (dtype == SA_BF16)
    for (int t : {(int)TQ, (int)TK, (int)TV, (int)TDO})
      if (a.st[t][2] >= (int64_t)1 << 24) return SA_ERR_UNSUPPORTED;
  a.row_ptr = row_ptr, a.col_idx = col_idx, a.col_ptr = col_ptr, a.row_idx = row_idx, a.sched = sched;
  a.col_capacity = col_capacity, a.row_capacity = row_capacity;
  a.nb = N / block, a.G = num_groups, a.mbs = mask_batch_stride, a.mhs = mask_head_stride, a.causal = causal;
  const bool bf = dtype == SA_BF16;
  if (!bf) {  // the bf16 dQ kernel computes the row statistics itself
    st = launch_delta(a, dtype, d, stream);
    if (st != SA_OK) return st;
  }
  if (d == 64) return block == 64 ? launch_bsa_bwd<64, 64>(a, bf, stream) : launch_bsa_bwd<64, 128>(a, bf, stream);
  return block == 64 ? launch_bsa_bwd<128, 64>(a, bf, stream) : launch_bsa_bwd<128, 128>(a, bf, stream);
}

extern "C" sa_status offset_attn_bwd(int32_t dtype, const void* q, const void* k, const void* v, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                     float* delta, int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                                     const int64_t* strides, const int32_t* offsets, int32_t num_offsets,
                                     float scale, hipStream_t stream) {
  BwdArgs a = {};
  if (!offsets) return SA_ERR_NULL;
  sa_status st = common_args(a, dtype, q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, strides, scale);
  if (st != SA_OK) return st;
  if (num_offsets < 1 || num_offsets > SA_MAX_OFFSETS) return SA_ERR_INVALID;
  for (int n = 0; n < num_offsets; ++n) {
    if (offsets[n] < 0 || offsets[n] >= N) return SA_ERR_INVALID;
    if (n > 0 && offsets[n] <= offsets[n - 1]) return SA_ERR_INVALID;
  }
  a.noff = num_offsets;
  for (int n = 0; n < num_offsets; ++n) a.offs[n] = offsets[n];
  st = launch_delta(a, dtype, d, stream);
  if (st != SA_OK) return st;
  const int64_t tiles = ((int64_t)N + 255) / 256;
  const int64_t nq = (int64_t)B * H * tiles, nk = (int64_t)B * H_kv * tiles;
  if (dtype == SA_BF16) {
    const int64_t t64 = ((int64_t)N + 63) / 64;
    const int64_t mq = (int64_t)B * H * t64, mk = (int64_t)B * H_kv * t64;
    st = d == 64 ? launch(off_bwd_dq_bf16<64>, a, mq, 256, 0, stream, "off_bwd_dq_bf16")
                 : launch(off_bwd_dq_bf16<128>, a, mq, 256, 0, stream, "off_bwd_dq_bf16");
    if (st != SA_OK) return st;
    return d == 64 ? launch(off_bwd_dkdv_bf16<64>, a, mk, 256, 0, stream, "off_bwd_dkdv_bf16")
                   : launch(off_bwd_dkdv_bf16<128>, a, mk, 256, 0, stream, "off_bwd_dkdv_bf16");
  }
  st = d == 64 ? launch(off_bwd_dq<64, false>, a, nq, 256, 0, stream, "off_bwd_dq")
               : launch(off_bwd_dq<128, false>, a, nq, 256, 0, stream, "off_bwd_dq");
  if (st != SA_OK) return st;
  return d == 64 ? launch(off_bwd_dkdv<64, false>, a, nk, 256, 0, stream, "off_bwd_dkdv")
                 : launch(off_bwd_dkdv<128, false>, a, nk, 256, 0, stream, "off_bwd_dkdv");
}
