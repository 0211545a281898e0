// Token-level offset attention ("Depth-Staggered Fibonacci Spacing for Sparse
// Attention", Sec. 2, "Attended set"): query t attends the keys t - delta for
// every distance delta of a table shared by all queries (a dense window
// {0..W} plus rounded scaled Fibonacci rungs), skipping t - delta < 0.
//
// The work per (query, key) is a single dot product and a single V update, so
// the kernel is bound by memory traffic, not by matrix throughput: one thread
// owns one query, keeps q and the fp32 accumulator in registers, and walks the
// table in chunks of 8 distances (8 dot products, one softmax rescale, 8 V
// updates).  Consecutive threads own consecutive queries, so for a fixed
// distance a wave reads one contiguous span of K / V rows.  Every K / V row is
// referenced by |table| different queries; those re-reads are served by L2:
// the workgroups of one head are mapped to one XCD (blockIdx % 8 selects the
// XCD) and the heads of an XCD are walked one after another.
#include <math.h>

#include <algorithm>
#include <vector>

#include "sa_device.h"
#include "sa_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;

struct OffArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs[3], ks[3], vs[3], os[3];
  int32_t B, H, H_kv, N, noff;
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

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void offset_fwd_kernel(OffArgs a) {
  typedef typename Elem<BF16>::T T;
  const int tiles = (a.N + kThreads - 1) / kThreads;
  const int BH = a.B * a.H;
  const int w = blockIdx.x;
  int bh, tile;
  if ((BH & 7) == 0) {  // keep all tiles of a head on one XCD
    const int xcd = w & 7, slot = w >> 3;
    bh = xcd + 8 * (slot / tiles);
    tile = slot % tiles;
  } else {
    bh = w / tiles;
    tile = w % tiles;
  }
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
  const dim3 grid((unsigned)((int64_t)B * H * tiles));
  if (dtype == SA_BF16) {
    if (d == 64)
      hipLaunchKernelGGL((offset_fwd_kernel<64, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((offset_fwd_kernel<128, true>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (d == 64)
      hipLaunchKernelGGL((offset_fwd_kernel<64, false>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((offset_fwd_kernel<128, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return sa_host::check_launch("offset_fwd_kernel");
}
