// Token-level offset attention ("Depth-Staggered Fibonacci Spacing for Sparse
// Attention", Sec. 2, "Attended set"): query t attends the keys t - delta for
// every distance delta of a table shared by all queries (a dense window
// {0..W} plus rounded scaled Fibonacci rungs), skipping t - delta < 0.
//
// Every (query, key) pair is a single dot product and a single V update, so
// the work is bound by moving K / V rows, not by matrix throughput.  bf16 path:
//   * a workgroup owns 64 consecutive queries of one head; four lanes share a
//     query, each holding a quarter of the head dimension, so the rows read for
//     a fixed distance form contiguous, fully used 64-byte segments and the
//     dot product needs only two quad (DPP) reductions;
//   * the near distances (<= 64) all read inside the span [t0 - R, t0 + 64)
//     (R = the largest near distance), which is staged once in LDS; the far
//     rungs are read straight from global memory / L2;
//   * distances are taken 8 at a time: 8 scores, one online-softmax rescale,
//     then V is accumulated two keys at a time with bf16 dot2 (the two keys'
//     values for one column are paired with a byte permute), one instruction
//     per two multiply-adds;
//   * workgroups of one head run on one XCD (blockIdx % 8 selects the XCD), so
//     every re-read of a K / V row by another query tile is served by its L2.
// fp32 path: one thread per query, plain fp32 arithmetic, for exact checks.
#include <math.h>

#include <algorithm>
#include <type_traits>
#include <vector>

#include "sa_device.h"
#include "sa_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;
constexpr int kNearMax = 64;   // distances up to this are served from the staged span

// Raise the dynamic-LDS limit of a kernel once (needed above 64 KiB).
inline sa_status allow_lds(const void* kern, int bytes) {
  if (bytes <= 65536) return SA_OK;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return e == hipSuccess ? SA_OK : sa_host::record_hip_error(e, "hipFuncSetAttribute");
}



struct OffArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs[3], ks[3], vs[3], os[3];
  int32_t B, H, H_kv, N, noff;
  int32_t nnear;  // offsets[0 .. nnear) are <= kNearMax and are read from the staged span
  int32_t span_r; // largest near offset (rows staged before the tile)
  float scale_log2;
  int32_t offs[SA_MAX_OFFSETS];
};

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

// Row of D elements -> D floats.
template <int D, bool BF16>
__device__ __forceinline__ void load_row(const typename Elem<BF16>::T* p, float* out) {
  if constexpr (BF16) {
#pragma unroll
    for (int x = 0; x < D; x += 8) {
      const sa::u32x4 w = *(const sa::u32x4*)(p + x);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[x + 2 * j] = sa::bf16_lo(w[j]);
        out[x + 2 * j + 1] = sa::bf16_hi(w[j]);
      }
    }
  } else {
#pragma unroll
    for (int x = 0; x < D; x += 4) {
      const sa::f32x4 w = *(const sa::f32x4*)(p + x);
      out[x] = w[0], out[x + 1] = w[1], out[x + 2] = w[2], out[x + 3] = w[3];
    }
  }
}

// (head, tile) of a workgroup; with B*H a multiple of 8 all tiles of a head go
// to one XCD (workgroup ids are dealt to the 8 XCDs round robin).
__device__ __forceinline__ void tile_of(int w, int BH, int tiles, int& bh, int& tile) {
  if ((BH & 7) == 0) {
    const int xcd = w & 7, slot = w >> 3;
    bh = xcd + 8 * (slot / tiles);
    tile = slot % tiles;
  } else {
    bh = w / tiles;
    tile = w % tiles;
  }
}

// 16-byte chunk slot inside a staged row (XOR swizzle against bank conflicts
// between the 16 rows one wave-instruction touches).
__device__ __forceinline__ int swz_row(int c, int row) { return c ^ (row & 7); }

// (v_a, v_b) bf16 pairs -> (lo halves), (hi halves)
__device__ __forceinline__ uint32_t pair_lo(uint32_t va, uint32_t vb) { return __builtin_amdgcn_perm(vb, va, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t va, uint32_t vb) { return __builtin_amdgcn_perm(vb, va, 0x07060302u); }

// Sum over the 4 lanes of a quad (DPP quad permutes, no LDS traffic).
__device__ __forceinline__ float quad_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  return x;
}

template <int D>
struct OffCfg {
  static constexpr int LPQ = 4;                 // lanes per query
  static constexpr int TQ = 64;                 // queries per workgroup
  static constexpr int NT = TQ * LPQ;           // threads
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int CPL = CPR / LPQ;         // chunks per lane: c = j + 4 m
  static constexpr int ROWB = D * 2;
  static constexpr int SPAN = TQ + kNearMax;    // staged rows
  static constexpr int LDSB = 2 * SPAN * ROWB;  // K and V
};

template <int D>
__global__ __launch_bounds__(256) void offset_bf16_kernel(OffArgs a) {
  using C = OffCfg<D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* ks = smem;
  uint8_t* vs = smem + C::SPAN * C::ROWB;

  const int tid = threadIdx.x;
  const int ql = tid / C::LPQ, j = tid % C::LPQ;
  const int tiles = (a.N + C::TQ - 1) / C::TQ;
  int bh, tile;
  tile_of(blockIdx.x, a.B * a.H, tiles, bh, tile);
  const int b = bh / a.H, h = bh % a.H, kvh = h / (a.H / a.H_kv);
  const int t0 = tile * C::TQ;
  const int t = t0 + ql;
  const bool live = t < a.N;
  const int tq = live ? t : a.N - 1;

  const uint16_t* Q = (const uint16_t*)a.q + b * a.qs[0] + h * a.qs[1];
  const char* Kb = (const char*)((const uint16_t*)a.k + b * a.ks[0] + kvh * a.ks[1]);
  const char* Vb = (const char*)((const uint16_t*)a.v + b * a.vs[0] + kvh * a.vs[1]);
  const uint32_t krow = (uint32_t)a.ks[2] * 2u, vrow = (uint32_t)a.vs[2] * 2u;  // bytes per row

  // stage rows [t0 - R, t0 + TQ) of K and V (rows outside [0, N) are skipped;
  // no query reads them)
  const int R = a.span_r;
  const int rows = C::TQ + R;
  for (int x = tid; x < rows * C::CPR; x += C::NT) {
    const int lr = x / C::CPR, c = x % C::CPR;
    const int r = t0 - R + lr;
    if (r < 0 || r >= a.N) continue;
    const int off = lr * C::ROWB + swz_row(c, lr) * 16;
    *(sa::u32x4*)(ks + off) = *(const sa::u32x4*)(Kb + (uint32_t)r * krow + 16u * c);
    *(sa::u32x4*)(vs + off) = *(const sa::u32x4*)(Vb + (uint32_t)r * vrow + 16u * c);
  }

  // this lane's quarter of q: chunks c = j + 4 m
  sa::u32x4 qv[C::CPL];
#pragma unroll
  for (int m = 0; m < C::CPL; ++m) qv[m] = *(const sa::u32x4*)(Q + (int64_t)tq * a.qs[2] + 8 * (j + 4 * m));
  float acc[C::CPL][8];
#pragma unroll
  for (int m = 0; m < C::CPL; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;
  __syncthreads();

  // One chunk of 8 distances [n0, n0 + 8) (entries past n1 repeat the range's
  // last distance and get weight 0): scores, one rescale, V update.  FAR rows
  // come from global memory, near ones from the staged span; MASKED: some
  // query of the tile precedes a distance of the chunk.
  auto chunk = [&](int n0, int n1, auto far_t, auto masked_t) {
    constexpr bool FAR = decltype(far_t)::value;
    constexpr bool MASKED = decltype(masked_t)::value;
    int src[kChunk];
    bool ok[kChunk];
#pragma unroll
    for (int cc = 0; cc < kChunk; ++cc) {
      const int delta = a.offs[min(n0 + cc, n1 - 1)];
      int s0 = tq - delta;
      ok[cc] = !MASKED || s0 >= 0;
      if (MASKED) s0 = max(s0, 0);
      src[cc] = FAR ? s0 : s0 - (t0 - R);  // global row, or row of the span
    }
    auto ld = [&](const char* g, const uint8_t* l, uint32_t grow, int cc, int m) -> sa::u32x4 {
      const int c = j + 4 * m;
      if (FAR) return *(const sa::u32x4*)(g + (uint32_t)src[cc] * grow + 16u * c);
      return *(const sa::u32x4*)(l + src[cc] * C::ROWB + swz_row(c, src[cc]) * 16);
    };
    float y[kChunk];
#pragma unroll
    for (int cc = 0; cc < kChunk; ++cc) {
      float dot = 0.f;
#pragma unroll
      for (int m = 0; m < C::CPL; ++m) {
        const sa::u32x4 kv = ld(Kb, ks, krow, cc, m);
#pragma unroll
        for (int w = 0; w < 4; ++w) dot = sa::dot2_bf16(qv[m][w], kv[w], dot);
      }
      dot = quad_sum(dot) * c2;
      y[cc] = (n0 + cc < n1 && ok[cc]) ? dot : -INFINITY;
    }
    float mx = y[0];
#pragma unroll
    for (int cc = 1; cc < kChunk; ++cc) mx = fmaxf(mx, y[cc]);
    if (mx > m_run) {  // per query (the quad agrees); rescale the running state
      const float alpha = sa::fast_exp2(m_run - mx);
      l_run *= alpha;
#pragma unroll
      for (int m = 0; m < C::CPL; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[m][e] *= alpha;
      m_run = mx;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int cc = 0; cc < kChunk; cc += 2) {
      const uint32_t pp = sa::pack_bf16x2(sa::fast_exp2(y[cc] - m_use), sa::fast_exp2(y[cc + 1] - m_use));
      l_run = sa::dot2_bf16(pp, 0x3f803f80u, l_run);
#pragma unroll
      for (int m = 0; m < C::CPL; ++m) {
        sa::u32x4 va = ld(Vb, vs, vrow, cc, m);
        sa::u32x4 vb = ld(Vb, vs, vrow, cc + 1, m);
        if (MASKED) {  // keys before the sequence start: zero weight and zero value
          if (!ok[cc]) va = sa::u32x4{0u, 0u, 0u, 0u};
          if (!ok[cc + 1]) vb = sa::u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[m][2 * w] = sa::dot2_bf16(pp, pair_lo(va[w], vb[w]), acc[m][2 * w]);
          acc[m][2 * w + 1] = sa::dot2_bf16(pp, pair_hi(va[w], vb[w]), acc[m][2 * w + 1]);
        }
      }
    }
  };

  // near distances from LDS, then far ones from global memory; a chunk needs
  // masking only if the tile's first query precedes its largest distance
  for (int n0 = 0; n0 < a.nnear; n0 += kChunk) {
    const int n1 = min(n0 + kChunk, a.nnear);
    if (t0 >= a.offs[n1 - 1])
      chunk(n0, n1, std::false_type{}, std::false_type{});
    else
      chunk(n0, n1, std::false_type{}, std::true_type{});
  }
  for (int n0 = a.nnear; n0 < a.noff; n0 += kChunk) {
    const int n1 = min(n0 + kChunk, a.noff);
    if (t0 >= a.offs[n1 - 1])
      chunk(n0, n1, std::true_type{}, std::false_type{});
    else
      chunk(n0, n1, std::true_type{}, std::true_type{});
  }

  if (!live) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* O = (uint16_t*)a.o + b * a.os[0] + h * a.os[1] + (int64_t)t * a.os[2];
#pragma unroll
  for (int m = 0; m < C::CPL; ++m) {
    sa::u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = sa::pack_bf16x2(acc[m][2 * e] * inv, acc[m][2 * e + 1] * inv);
    *(sa::u32x4*)(O + 8 * (j + 4 * m)) = w;
  }
  if (j == 0) a.lse[((int64_t)b * a.H + h) * a.N + t] = l_run > 0.f ? (m_run + log2f(l_run)) * sa::kLn2 : -INFINITY;
}

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void offset_fwd_kernel(OffArgs a) {
  typedef typename Elem<BF16>::T T;
  const int tiles = (a.N + kThreads - 1) / kThreads;
  int bh, tile;
  tile_of(blockIdx.x, a.B * a.H, tiles, bh, tile);
  const int b = bh / a.H, h = bh % a.H, kvh = h / (a.H / a.H_kv);
  const int t = tile * kThreads + threadIdx.x;
  if (t >= a.N) return;

  const T* Q = (const T*)a.q + b * a.qs[0] + h * a.qs[1];
  const T* K = (const T*)a.k + b * a.ks[0] + kvh * a.ks[1];
  const T* V = (const T*)a.v + b * a.vs[0] + kvh * a.vs[1];
  T* O = (T*)a.o + b * a.os[0] + h * a.os[1];

  float qf[D], acc[D];
  load_row<D, BF16>(Q + (int64_t)t * a.qs[2], qf);
#pragma unroll
  for (int x = 0; x < D; ++x) acc[x] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c2 = a.scale_log2;

  // the table is ascending: once t - delta < 0 every later distance is too
  int nvalid = 0;
  while (nvalid < a.noff && a.offs[nvalid] <= t) ++nvalid;

  for (int n0 = 0; n0 < nvalid; n0 += kChunk) {
    float y[kChunk];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      y[c] = -INFINITY;
      if (n0 + c < nvalid) {
        const int64_t src = t - a.offs[n0 + c];
        float kf[D];
        load_row<D, BF16>(K + src * a.ks[2], kf);
        float dot = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) dot = fmaf(qf[x], kf[x], dot);
        y[c] = dot * c2;
        mx = fmaxf(mx, y[c]);
      }
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = sa::fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int x = 0; x < D; ++x) acc[x] *= alpha;
    m = m_new;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      if (n0 + c < nvalid) {
        const float p = sa::fast_exp2(y[c] - m);
        l += p;
        const int64_t src = t - a.offs[n0 + c];
        float vf[D];
        load_row<D, BF16>(V + src * a.vs[2], vf);
#pragma unroll
        for (int x = 0; x < D; ++x) acc[x] = fmaf(p, vf[x], acc[x]);
      }
    }
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* orow = O + (int64_t)t * a.os[2];
  if constexpr (BF16) {
#pragma unroll
    for (int x = 0; x < D; x += 8) {
      sa::u32x4 wv;
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = sa::pack_bf16x2(acc[x + 2 * j] * inv, acc[x + 2 * j + 1] * inv);
      *(sa::u32x4*)(orow + x) = wv;
    }
  } else {
#pragma unroll
    for (int x = 0; x < D; x += 4) {
      sa::f32x4 wv = {acc[x] * inv, acc[x + 1] * inv, acc[x + 2] * inv, acc[x + 3] * inv};
      *(sa::f32x4*)(orow + x) = wv;
    }
  }
  a.lse[((int64_t)b * a.H + h) * a.N + t] = l > 0.f ? (m + log2f(l)) * sa::kLn2 : -INFINITY;
}

}  // namespace

extern "C" sa_status offset_attn_make_table(int32_t W, double alpha, const int64_t* base, int32_t K,
                                            int32_t N, int32_t* table_out, int32_t capacity,
                                            int32_t* count_out) {
#pragma clang fp contract(off)
  if (!table_out || !count_out || (K > 0 && !base)) return SA_ERR_NULL;
  if (W < 0 || K < 0 || N < 1 || capacity < 0 || !isfinite(alpha)) return SA_ERR_INVALID;
  std::vector<int64_t> d;
  for (int64_t x = 0; x <= W && x < N; ++x) d.push_back(x);
  for (int k = 0; k < K; ++k) {
    if (base[k] < 0) return SA_ERR_INVALID;
    const double prod = alpha * (double)base[k];  // rounded product, then + 1/2
    const double x = floor(prod + 0.5);
    if (x >= 0.0 && x < (double)N) d.push_back((int64_t)x);
  }
  std::sort(d.begin(), d.end());
  d.erase(std::unique(d.begin(), d.end()), d.end());
  if ((int64_t)d.size() > capacity) return SA_ERR_CAPACITY;
  for (size_t j = 0; j < d.size(); ++j) table_out[j] = (int32_t)d[j];
  *count_out = (int32_t)d.size();
  return SA_OK;
}

extern "C" sa_status offset_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                                     void* o, float* lse, int32_t B, int32_t H, int32_t H_kv,
                                     int32_t N, int32_t d, const int64_t* strides,
                                     const int32_t* offsets, int32_t num_offsets, float scale,
                                     hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !offsets) return SA_ERR_NULL;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_INVALID;
  if (B < 1 || H < 1 || H_kv < 1 || N < 1 || d < 1) return SA_ERR_INVALID;
  if (H % H_kv != 0) return SA_ERR_INVALID;
  if (!isfinite(scale)) return SA_ERR_INVALID;
  if (num_offsets < 1 || num_offsets > SA_MAX_OFFSETS) return SA_ERR_INVALID;
  for (int n = 0; n < num_offsets; ++n) {
    if (offsets[n] < 0 || offsets[n] >= N) return SA_ERR_INVALID;
    if (n > 0 && offsets[n] <= offsets[n - 1]) return SA_ERR_INVALID;
  }
  if (d != 64 && d != 128) return SA_ERR_UNSUPPORTED;
  const int64_t tiles = ((int64_t)N + kThreads - 1) / kThreads;
  if ((int64_t)B * H * tiles > 0x7fffffffll) return SA_ERR_UNSUPPORTED;
  if (!sa_host::aligned16(q) || !sa_host::aligned16(k) || !sa_host::aligned16(v) ||
      !sa_host::aligned16(o))
    return SA_ERR_INVALID;
  sa_host::Strides st[4];
  const sa_status ss = sa_host::resolve_strides(strides, B, H, H_kv, N, d, dtype == SA_BF16 ? 8 : 4, st);
  if (ss != SA_OK) return ss;

  OffArgs a = {};
  a.q = q, a.k = k, a.v = v, a.o = o, a.lse = lse;
  int64_t* dst[4] = {a.qs, a.ks, a.vs, a.os};
  for (int t = 0; t < 4; ++t) dst[t][0] = st[t].b, dst[t][1] = st[t].h, dst[t][2] = st[t].s;
  a.B = B, a.H = H, a.H_kv = H_kv, a.N = N, a.noff = num_offsets;
  a.scale_log2 = scale * sa::kLog2e;
  for (int n = 0; n < num_offsets; ++n) a.offs[n] = offsets[n];
  a.nnear = 0;
  a.span_r = 0;
  while (a.nnear < num_offsets && offsets[a.nnear] <= kNearMax) a.span_r = offsets[a.nnear++];
  if (dtype == SA_BF16) {
    if (d == 64) {
      using Cf = OffCfg<64>;
      static const sa_status lds_ok = allow_lds((const void*)&offset_bf16_kernel<64>, Cf::LDSB);
      if (lds_ok != SA_OK) return lds_ok;
      const dim3 grid((unsigned)((int64_t)B * H * ((N + Cf::TQ - 1) / Cf::TQ)));
      hipLaunchKernelGGL((offset_bf16_kernel<64>), grid, dim3(Cf::NT), Cf::LDSB, stream, a);
    } else {
      using Cf = OffCfg<128>;
      static const sa_status lds_ok = allow_lds((const void*)&offset_bf16_kernel<128>, Cf::LDSB);
      if (lds_ok != SA_OK) return lds_ok;
      const dim3 grid((unsigned)((int64_t)B * H * ((N + Cf::TQ - 1) / Cf::TQ)));
      hipLaunchKernelGGL((offset_bf16_kernel<128>), grid, dim3(Cf::NT), Cf::LDSB, stream, a);
    }
  } else {
    const dim3 grid((unsigned)((int64_t)B * H * tiles));
    if (d == 64)
      hipLaunchKernelGGL((offset_fwd_kernel<64, false>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((offset_fwd_kernel<128, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return sa_host::check_launch("offset_fwd_kernel");
}
