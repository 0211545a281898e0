// Block-sparse attention forward over a CSR list of key blocks.
//
// What is computed ("Parameter-free Adaptive Sparse Attention via
// Compression-Based Content Selection", Sec. 3.4 block-to-token expansion and
// Appendix B Algorithm 1 step 4; "BigBird", Sec. 3): masked softmax attention
// where query t sees the tokens of the key blocks listed for its query block,
// restricted to s <= t when causal.  The token mask is never built: blocks that
// are not listed are never touched, and the causal triangle is applied only on
// the diagonal block.
//
// bf16 path (MFMA, gfx950):
//   * one workgroup per (batch, head, query block); one wave per 32 queries;
//   * key blocks are walked in 64-key sub-tiles; K (row-major) and V (stored
//     transposed) of the next sub-tile are fetched into registers while the
//     current one is consumed from LDS (two LDS stages, one barrier per step);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16, so every lane owns one query
//     column: the row max / sum of the online softmax are in-lane except for a
//     single exchange with lane ^ 32;
//   * O^T += V^T P^T on the same MFMA: the fp32 accumulator of S^T already holds
//     exactly the keys each lane must supply as the P operand, so P goes from
//     the accumulator to the operand registers with one bf16 pack and no LDS
//     round trip.  V is written to LDS transposed, with key bits 2 and 3 swapped
//     so that each lane reads its 8 keys as one 16-byte word;
//   * 16-byte LDS chunks are XOR-swizzled so the MFMA operand reads and the
//     staging writes are free of bank conflicts;
//   * launch order follows `sched` (longest rows first); blockIdx % (B*H) picks
//     the head, so with B*H a multiple of 8 every query block of one head runs
//     on the same XCD and shares its L2.
// fp32 path: a plain VALU kernel, one thread per query, for exact checks.
#include <math.h>

#include "sa_device.h"
#include "sa_host.h"

namespace {

struct BsaArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs[3], ks[3], vs[3], os[3];  // batch, head, seq strides (elements)
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t col_capacity;
  const int32_t* sched;
  int32_t B, H, H_kv, N, nb, G;
  int64_t mbs, mhs;
  int32_t causal;
  float scale;       // logit scale
  float scale_log2;  // scale * log2(e)
};

// Work item of a workgroup: head (b, h), query block i, CSR entry range.
struct Item {
  int32_t b, h, kvh, i;
  int64_t e_beg, e_end;
  bool ok;
};

__device__ __forceinline__ Item work_item(const BsaArgs& a) {
  Item it;
  const int32_t BH = a.B * a.H;
  const int32_t w = blockIdx.x;
  const int32_t pos = w / BH, bh = w - pos * BH;
  it.b = bh / a.H;
  it.h = bh - it.b * a.H;
  it.kvh = it.h / (a.H / a.H_kv);
  const int64_t g = (int64_t)it.b * a.mbs + (int64_t)it.h * a.mhs;
  it.i = a.sched ? a.sched[g * a.nb + pos] : pos;
  it.ok = it.i >= 0 && it.i < a.nb;
  const int64_t r = g * a.nb + (it.ok ? it.i : 0);
  int64_t e0 = a.row_ptr[r], e1 = a.row_ptr[r + 1];
  e0 = max((int64_t)0, min(e0, a.col_capacity));
  e1 = max(e0, min(e1, a.col_capacity));
  it.e_beg = e0;
  it.e_end = e1;
  return it;
}

// First CSR entry at or after e whose block is usable (in range, and not after
// the query block when causal).  Uniform across the workgroup.
__device__ __forceinline__ int64_t next_entry(const BsaArgs& a, const Item& it, int64_t e) {
  for (; e < it.e_end; ++e) {
    const int32_t kb = a.col_idx[e];
    if (kb >= 0 && kb < a.nb && !(a.causal && kb > it.i)) break;
  }
  return e;
}

// ---------------------------------------------------------------- bf16 ----

__device__ __forceinline__ int swz_k(int c, int key) { return (c & ~7) | ((c ^ key) & 7); }
__device__ __forceinline__ int swz_v(int d) { return (d ^ (d >> 3)) & 7; }
// position of key (0..63) inside a transposed V row: bits 2 and 3 swapped
__device__ __forceinline__ int vpos_of_quad(int k4) {  // k4 = key / 4
  return 4 * ((k4 & ~3) | ((k4 & 1) << 1) | ((k4 >> 1) & 1));
}

template <int D, int BLK>
struct BsaCfg {
  static constexpr int NW = BLK / 32;        // waves per workgroup
  static constexpr int NT = NW * 64;         // threads
  static constexpr int SUBS = BLK / 64;      // 64-key sub-tiles per key block
  static constexpr int KROW = D * 2;         // bytes per K row in LDS
  static constexpr int KTILE = 64 * KROW;    // K sub-tile bytes
  static constexpr int VTILE = D * 128;      // V^T sub-tile bytes (D rows of 64 keys)
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int KU = (8 * D + NT - 1) / NT;  // 16-byte K chunks per thread
  static constexpr int VU = (2 * D + NT - 1) / NT;  // 4-key x 8-d V units per thread
};

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void bsa_fwd_bf16_kernel(BsaArgs a) {
  using C = BsaCfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, lq = lane & 31;
  const Item it = work_item(a);
  if (!it.ok) return;

  const uint16_t* Q = (const uint16_t*)a.q + it.b * a.qs[0] + it.h * a.qs[1];
  const uint16_t* K = (const uint16_t*)a.k + it.b * a.ks[0] + it.kvh * a.ks[1];
  const uint16_t* V = (const uint16_t*)a.v + it.b * a.vs[0] + it.kvh * a.vs[1];
  uint16_t* O = (uint16_t*)a.o + it.b * a.os[0] + it.h * a.os[1];
  float* L = a.lse + ((int64_t)it.b * a.H + it.h) * a.N;

  const int q_local = wave * 32 + lq;
  const int64_t qpos = (int64_t)it.i * BLK + q_local;

  // Q^T as the B operand: lane holds query lq, d = 16 ks + 8 hl .. + 7
  sa::u32x4 qr[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qr[ks] = *(const sa::u32x4*)(Q + qpos * a.qs[2] + 16 * ks + 8 * hl);

  sa::f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  sa::u32x4 kreg[C::KU];
  sa::u32x4 vreg[C::VU][4];

  auto load_tile = [&](int32_t kb, int s) {
    const int64_t key0 = (int64_t)kb * BLK + 64 * s;
#pragma unroll
    for (int x = 0; x < C::KU; ++x) {
      const int u = tid + x * C::NT;
      if (u < 8 * D) {
        const int key = u / (D / 8), c = u % (D / 8);
        kreg[x] = *(const sa::u32x4*)(K + (key0 + key) * a.ks[2] + 8 * c);
      }
    }
#pragma unroll
    for (int x = 0; x < C::VU; ++x) {
      const int u = tid + x * C::NT;
      if (u < 2 * D) {
        const int k4 = u / (D / 8), c = u % (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          vreg[x][rr] = *(const sa::u32x4*)(V + (key0 + 4 * k4 + rr) * a.vs[2] + 8 * c);
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint8_t* Kb = smem + buf * C::STAGE;
    uint8_t* Vb = Kb + C::KTILE;
#pragma unroll
    for (int x = 0; x < C::KU; ++x) {
      const int u = tid + x * C::NT;
      if (u < 8 * D) {
        const int key = u / (D / 8), c = u % (D / 8);
        *(sa::u32x4*)(Kb + key * C::KROW + swz_k(c, key) * 16) = kreg[x];
      }
    }
#pragma unroll
    for (int x = 0; x < C::VU; ++x) {
      const int u = tid + x * C::NT;
      if (u < 2 * D) {
        const int k4 = u / (D / 8), c = u % (D / 8);
        const int pos = vpos_of_quad(k4);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int d = 8 * c + dd;
          const int wi = dd >> 1;
          uint32_t w0, w1;
          if (dd & 1) {
            w0 = (vreg[x][0][wi] >> 16) | (vreg[x][1][wi] & 0xffff0000u);
            w1 = (vreg[x][2][wi] >> 16) | (vreg[x][3][wi] & 0xffff0000u);
          } else {
            w0 = (vreg[x][0][wi] & 0xffffu) | (vreg[x][1][wi] << 16);
            w1 = (vreg[x][2][wi] & 0xffffu) | (vreg[x][3][wi] << 16);
          }
          sa::u32x2 val = {w0, w1};
          *(sa::u32x2*)(Vb + d * 128 + (((pos >> 3) ^ swz_v(d)) << 4) + (pos & 7) * 2) = val;
        }
      }
    }
  };

  const float c2 = a.scale_log2;

  auto compute_tile = [&](int buf, int32_t kb, int s) {
    const bool diag = a.causal && kb == it.i;
    const int sub_local = 64 * s;
    if (diag && sub_local > wave * 32 + 31) return;  // whole sub-tile after these queries
    const bool need_mask = diag && (sub_local + 63 > wave * 32);
    const uint8_t* Kb = smem + buf * C::STAGE;
    const uint8_t* Vb = Kb + C::KTILE;

    sa::f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = 32 * kt + lq;
        const sa::u32x4 av = *(const sa::u32x4*)(Kb + key * C::KROW + swz_k(2 * ks + hl, key) * 16);
        sacc[kt] = sa::mfma32(av, qr[ks], sacc[kt]);
      }
    }

    // scaled logits (log2 units); masked -> -inf
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float y = sacc[kt][e] * c2;
        if (need_mask) {
          const int key_local = sub_local + 32 * kt + 8 * (e >> 2) + 4 * hl + (e & 3);
          if (key_local > q_local) y = -INFINITY;
        }
        sacc[kt][e] = y;
        mx = fmaxf(mx, y);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = sa::fast_exp2(m_run - m_use);
    float lsum = 0.f;
    sa::u32x4 pb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = sa::fast_exp2(sacc[kt][e] - m_use);
        lsum += p[e];
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int w = 0; w < 4; ++w) pb[kt][t][w] = sa::pack_bf16x2(p[8 * t + 2 * w], p[8 * t + 2 * w + 1]);
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;

#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int d = 32 * dt + lq;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const sa::u32x4 av = *(const sa::u32x4*)(Vb + d * 128 + (((2 * u + hl) ^ swz_v(d)) << 4));
        oacc[dt] = sa::mfma32(av, pb[u >> 1][u & 1], oacc[dt]);
      }
    }
  };

  // walk the sub-tiles: prefetch n+1 into registers while n is consumed from LDS
  int64_t e = next_entry(a, it, it.e_beg);
  int s = 0;
  if (e < it.e_end) {
    load_tile(a.col_idx[e], 0);
    store_tile(0);
  }
  __syncthreads();
  int buf = 0;
  while (e < it.e_end) {
    const int32_t kb = a.col_idx[e];
    int64_t e2 = e;
    int s2 = s + 1;
    if (s2 == C::SUBS) {
      s2 = 0;
      e2 = next_entry(a, it, e + 1);
    }
    const bool has_next = e2 < it.e_end;
    if (has_next) load_tile(a.col_idx[e2], s2);
    compute_tile(buf, kb, s);
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    e = e2;
    s = s2;
  }

  // finalise: combine the two half-rows of each query, normalise, store
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* orow = O + qpos * a.os[2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d0 = 32 * dt + 8 * ii + 4 * hl;
      sa::u32x2 w = {sa::pack_bf16x2(oacc[dt][4 * ii + 0] * inv, oacc[dt][4 * ii + 1] * inv),
                     sa::pack_bf16x2(oacc[dt][4 * ii + 2] * inv, oacc[dt][4 * ii + 3] * inv)};
      *(sa::u32x2*)(orow + d0) = w;
    }
  if (hl == 0) L[qpos] = l_tot > 0.f ? (m_run + log2f(l_tot)) * sa::kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- fp32 ----

template <int D, int BLK>
__global__ __launch_bounds__(BLK) void bsa_fwd_f32_kernel(BsaArgs a) {
  __shared__ __attribute__((aligned(16))) float ksm[64][D];
  __shared__ __attribute__((aligned(16))) float vsm[64][D];
  const int tid = threadIdx.x;
  const Item it = work_item(a);
  if (!it.ok) return;
  const float* Q = (const float*)a.q + it.b * a.qs[0] + it.h * a.qs[1];
  const float* K = (const float*)a.k + it.b * a.ks[0] + it.kvh * a.ks[1];
  const float* V = (const float*)a.v + it.b * a.vs[0] + it.kvh * a.vs[1];
  float* O = (float*)a.o + it.b * a.os[0] + it.h * a.os[1];
  float* L = a.lse + ((int64_t)it.b * a.H + it.h) * a.N;
  const int64_t qpos = (int64_t)it.i * BLK + tid;

  float qv[D], acc[D];
#pragma unroll
  for (int x = 0; x < D; x += 4) {
    const sa::f32x4 t = *(const sa::f32x4*)(Q + qpos * a.qs[2] + x);
    qv[x] = t[0], qv[x + 1] = t[1], qv[x + 2] = t[2], qv[x + 3] = t[3];
    acc[x] = acc[x + 1] = acc[x + 2] = acc[x + 3] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int64_t e = next_entry(a, it, it.e_beg); e < it.e_end; e = next_entry(a, it, e + 1)) {
    const int32_t kb = a.col_idx[e];
    const bool diag = a.causal && kb == it.i;
    for (int s = 0; s < BLK / 64; ++s) {
      const int64_t key0 = (int64_t)kb * BLK + 64 * s;
      __syncthreads();
      for (int u = tid; u < 64 * D / 4; u += BLK) {
        const int key = u / (D / 4), c = u % (D / 4);
        *(sa::f32x4*)&ksm[key][4 * c] = *(const sa::f32x4*)(K + (key0 + key) * a.ks[2] + 4 * c);
        *(sa::f32x4*)&vsm[key][4 * c] = *(const sa::f32x4*)(V + (key0 + key) * a.vs[2] + 4 * c);
      }
      __syncthreads();
      for (int kk = 0; kk < 64; ++kk) {
        if (diag && 64 * s + kk > tid) break;
        float dot = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) dot = fmaf(qv[x], ksm[kk][x], dot);
        const float y = dot * a.scale;
        if (y > m) {
          const float al = expf(m - y);
          l *= al;
#pragma unroll
          for (int x = 0; x < D; ++x) acc[x] *= al;
          m = y;
        }
        const float p = expf(y - m);
        l += p;
#pragma unroll
        for (int x = 0; x < D; ++x) acc[x] = fmaf(p, vsm[kk][x], acc[x]);
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int x = 0; x < D; x += 4) {
    sa::f32x4 t = {acc[x] * inv, acc[x + 1] * inv, acc[x + 2] * inv, acc[x + 3] * inv};
    *(sa::f32x4*)(O + qpos * a.os[2] + x) = t;
  }
  L[qpos] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <typename Kern>
sa_status launch(Kern kern, const BsaArgs& a, int threads, hipStream_t stream, const char* name) {
  const int64_t grid = (int64_t)a.B * a.H * a.nb;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return sa_host::check_launch(name);
}

}  // namespace

extern "C" sa_status sparse_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                                     void* o, float* lse, int32_t B, int32_t H, int32_t H_kv,
                                     int32_t N, int32_t d, int32_t block, const int64_t* strides,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t col_capacity, const int32_t* sched, int32_t num_groups,
                                     int64_t mask_batch_stride, int64_t mask_head_stride,
                                     int32_t causal, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !row_ptr || !col_idx) return SA_ERR_NULL;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_INVALID;
  if (B < 1 || H < 1 || H_kv < 1 || N < 1 || d < 1 || block < 1) return SA_ERR_INVALID;
  if (H % H_kv != 0) return SA_ERR_INVALID;
  if (causal != 0 && causal != 1) return SA_ERR_INVALID;
  if (!isfinite(scale)) return SA_ERR_INVALID;
  if (col_capacity < 0) return SA_ERR_INVALID;
  if (num_groups < 1 || mask_batch_stride < 0 || mask_head_stride < 0) return SA_ERR_INVALID;
  if ((int64_t)(B - 1) * mask_batch_stride + (int64_t)(H - 1) * mask_head_stride >= num_groups)
    return SA_ERR_INVALID;
  if (N % block != 0) return SA_ERR_INVALID;
  if ((d != 64 && d != 128) || (block != 64 && block != 128)) return SA_ERR_UNSUPPORTED;
  const int64_t nb = N / block;
  if ((int64_t)B * H * nb > 0x7fffffffll) return SA_ERR_UNSUPPORTED;
  if (!sa_host::aligned16(q) || !sa_host::aligned16(k) || !sa_host::aligned16(v) ||
      !sa_host::aligned16(o))
    return SA_ERR_INVALID;
  sa_host::Strides st[4];
  const sa_status ss = sa_host::resolve_strides(strides, B, H, H_kv, N, d, dtype == SA_BF16 ? 8 : 4, st);
  if (ss != SA_OK) return ss;

  BsaArgs a = {};
  a.q = q, a.k = k, a.v = v, a.o = o, a.lse = lse;
  int64_t* dst[4] = {a.qs, a.ks, a.vs, a.os};
  for (int t = 0; t < 4; ++t) dst[t][0] = st[t].b, dst[t][1] = st[t].h, dst[t][2] = st[t].s;
  a.row_ptr = row_ptr, a.col_idx = col_idx, a.col_capacity = col_capacity, a.sched = sched;
  a.B = B, a.H = H, a.H_kv = H_kv, a.N = N, a.nb = (int32_t)nb, a.G = num_groups;
  a.mbs = mask_batch_stride, a.mhs = mask_head_stride;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * sa::kLog2e;

  if (dtype == SA_BF16) {
    if (d == 64 && block == 64) return launch(bsa_fwd_bf16_kernel<64, 64>, a, 128, stream, "bsa_fwd_bf16<64,64>");
    if (d == 64 && block == 128) return launch(bsa_fwd_bf16_kernel<64, 128>, a, 256, stream, "bsa_fwd_bf16<64,128>");
    if (d == 128 && block == 64) return launch(bsa_fwd_bf16_kernel<128, 64>, a, 128, stream, "bsa_fwd_bf16<128,64>");
    return launch(bsa_fwd_bf16_kernel<128, 128>, a, 256, stream, "bsa_fwd_bf16<128,128>");
  }
  if (d == 64 && block == 64) return launch(bsa_fwd_f32_kernel<64, 64>, a, 64, stream, "bsa_fwd_f32<64,64>");
  if (d == 64 && block == 128) return launch(bsa_fwd_f32_kernel<64, 128>, a, 128, stream, "bsa_fwd_f32<64,128>");
  if (d == 128 && block == 64) return launch(bsa_fwd_f32_kernel<128, 64>, a, 64, stream, "bsa_fwd_f32<128,64>");
  return launch(bsa_fwd_f32_kernel<128, 128>, a, 128, stream, "bsa_fwd_f32<128,128>");
}
