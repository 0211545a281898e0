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
//
// Workgroup = NP groups of BLK/32 waves.  Every group covers all BLK queries
// of the query block (one wave per 32 queries) and takes every NP-th 64-key
// tile of the row; the groups' partial softmax states are merged through LDS
// at the end.  K / V tiles travel global -> LDS with direct (DMA) loads into an
// S-stage ring, so no registers are spent on staging and the loads of later
// tiles overlap the MFMAs of the current one.  The row's key-block ids are
// copied to LDS first, so the loop itself issues no global loads besides the
// DMA (the explicit vmcnt waits then count only tile loads).

// Workgroup barrier that does not drain outstanding DMA loads (a fenced
// barrier would wait for every in-flight tile, not just the one needed).
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte chunk position inside a K row: XOR with the key's low bits so the
// 32 rows read by one MFMA operand load fall into distinct bank groups.
__device__ __forceinline__ int swz_k(int c, int key) { return c ^ (key & 7); }
// ... and inside a V row, matched to the 4-row groups of the transpose read.
__device__ __forceinline__ int swz_v(int c, int key) { return c ^ ((key & 3) << 1); }

template <int D, int BLK, int NP, int S>
struct BsaCfg {
  static constexpr int QW = BLK / 32;               // waves per group
  static constexpr int NW = QW * NP;                // waves per workgroup
  static constexpr int NT = NW * 64;                // threads
  static constexpr int SUBS = BLK / 64;             // 64-key tiles per key block
  static constexpr int CPR = D / 8;                 // 16-byte chunks per K / V row
  static constexpr int ROWB = D * 2;                // bytes per K / V row
  static constexpr int KVB = 64 * ROWB;             // bytes of one K (or V) tile
  static constexpr int TILEB = 2 * KVB;             // K + V
  static constexpr int STAGEB = NP * TILEB;
  static constexpr int LIST = 256;                  // key-block ids held in LDS at once
  static constexpr int LDSB = S * STAGEB + LIST * 4;
  static constexpr int CHUNKS = TILEB / 16;         // 16-byte chunks per tile
  static constexpr int LPI = NP * CHUNKS / NT;      // DMA loads per thread per stage
  static_assert(S >= 2 && S <= 3, "2 or 3 stages");
  // merge area: per (group > 0, wave, lane): O^T partial (D/2 floats), m, l
  static constexpr int MERGEB = (NP - 1) * QW * 64 * (D / 2 + 2) * 4;
  static_assert(MERGEB <= S * STAGEB, "merge area must fit in the ring");
};

template <int D, int BLK, int NP, int S>
__global__ __launch_bounds__(BLK / 32 * NP * 64) void bsa_fwd_bf16_kernel(BsaArgs a) {
  using C = BsaCfg<D, BLK, NP, S>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t* list = (int32_t*)(smem + S * C::STAGEB);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = sa::uniform(tid >> 6);
  const int grp = wave / C::QW, wq = wave % C::QW;
  const int hl = lane >> 5, lq = lane & 31;
  const Item it = work_item(a);
  if (!it.ok) return;

  const uint16_t* Q = (const uint16_t*)a.q + it.b * a.qs[0] + it.h * a.qs[1];
  const uint16_t* K = (const uint16_t*)a.k + it.b * a.ks[0] + it.kvh * a.ks[1];
  const uint16_t* V = (const uint16_t*)a.v + it.b * a.vs[0] + it.kvh * a.vs[1];
  const int64_t ks2 = a.ks[2], vs2 = a.vs[2];
  const int32_t limit = a.causal ? it.i + 1 : a.nb;  // usable key blocks are < limit

  // Q^T as the B operand: lane holds query lq of this wave, d = 16 k + 8 hl .. +7
  const int q_local = wq * 32 + lq;
  const int64_t qpos = (int64_t)it.i * BLK + q_local;
  sa::u32x4 qr[D / 16];
#pragma unroll
  for (int k = 0; k < D / 16; ++k) qr[k] = *(const sa::u32x4*)(Q + qpos * a.qs[2] + 16 * k + 8 * hl);
  // Consume Q here so the compiler's own load wait happens once, before the
  // loop, and not inside it where it would also wait for the tile prefetch.
#pragma unroll
  for (int k = 0; k < D / 16; ++k) asm volatile("" ::"v"(qr[k]));

  sa::f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_used = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;
  constexpr float kTau = 8.f;  // rescale only when the running max grows by > 2^8

  // DMA plan: for each tile of a stage, K and V (KVB bytes each) are copied by
  // JN wave-instructions per thread; instruction j of wave w covers chunks
  // [j*NT + 64 w, j*NT + 64 w + 64) of the K (or V) tile, i.e. whole rows.
  // The lane part of each swizzled source offset is fixed for the kernel.
  constexpr int JN = (C::CHUNKS / 2) / C::NT;
  static_assert((C::CHUNKS / 2) % C::NT == 0, "K / V tiles must split evenly over the threads");
  uint32_t offK[JN], offV[JN];
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int r = j * C::NT + wave * 64 + lane;  // chunk of this lane
    const int key = r / C::CPR, cs = r % C::CPR;
    offK[j] = (uint32_t)(key * ks2 * 2) + 16u * (uint32_t)swz_k(cs, key);
    offV[j] = (uint32_t)(key * vs2 * 2) + 16u * (uint32_t)swz_v(cs, key);
  }

  for (int64_t base = it.e_beg; base < it.e_end; base += C::LIST) {
    const int cnt = (int)min((int64_t)C::LIST, it.e_end - base);
    __syncthreads();  // previous pass finished with the list and the ring
    for (int x = tid; x < cnt; x += C::NT) list[x] = a.col_idx[base + x];
    __syncthreads();
    const int T = cnt * C::SUBS;        // 64-key tiles of this pass
    const int NI = (T + NP - 1) / NP;   // pipeline iterations

    // key block of tile t (t clamped into the pass); ids outside [0, limit)
    // are replaced by a safe block and the tile is skipped at compute time
    auto tile_kb = [&](int t, bool& ok) -> int32_t {
      const int32_t kb = sa::uniform(list[min(t, T - 1) / C::SUBS]);
      ok = kb >= 0 && kb < limit;
      return ok ? kb : it.i;
    };

    auto issue_stage = [&](int n) {  // DMA loads of iteration n into stage n % S
      uint8_t* st = smem + (n % S) * C::STAGEB;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        bool ok;
        const int t = min(n * NP + p, T - 1);
        const int64_t key0 = (int64_t)tile_kb(t, ok) * BLK + 64 * (t % C::SUBS);
        const char* kbase = (const char*)(K + key0 * ks2);
        const char* vbase = (const char*)(V + key0 * vs2);
        uint8_t* kdst = st + p * C::TILEB + wave * 64 * 16;
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          // wave-uniform LDS base; lane i lands at base + 16 i
          sa::dma16(kbase + offK[j], kdst + j * C::NT * 16);
          sa::dma16(vbase + offV[j], kdst + C::KVB + j * C::NT * 16);
        }
      }
    };

    if (NI > 0) issue_stage(0);
    if (S == 3 && NI > 1) issue_stage(1);

    for (int n = 0; n < NI; ++n) {
      if (S == 3 && n + 1 < NI)
        wait_vmcnt<C::LPI>();
      else
        wait_vmcnt<0>();
      ring_barrier();  // stage n is complete for every wave; stage n-1 is free
      if (n + S - 1 < NI) issue_stage(n + S - 1);

      const int t = n * NP + grp;
      bool ok;
      const int32_t kb = tile_kb(t, ok);
      const int sub = t % C::SUBS;
      const bool diag = a.causal && kb == it.i;
      const int sub_local = 64 * sub;
      if (!(t < T && ok && !(diag && sub_local > wq * 32 + 31))) continue;

      const uint8_t* Ks = smem + (n % S) * C::STAGEB + grp * C::TILEB;
      const uint8_t* Vs = Ks + C::KVB;
      // S^T = K Q^T for 64 keys x 32 queries
      sa::f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
#pragma unroll
      for (int k = 0; k < D / 16; ++k)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int key = 32 * kt + lq;
          const sa::u32x4 av = *(const sa::u32x4*)(Ks + key * C::ROWB + swz_k(2 * k + hl, key) * 16);
          sacc[kt] = sa::mfma32(av, qr[k], sacc[kt]);
        }
      // Diagonal tile: keys after the query are replaced by a logit that
      // scales to -inf (the sign of c2 picks it; c2 is never 0), so the common
      // path below needs no per-element select.
      if (diag && (sub_local + 63 > wq * 32)) {
        const float masked = c2 > 0.f ? -INFINITY : INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key_local = sub_local + 32 * kt + 8 * (e >> 2) + 4 * hl + (e & 3);
            if (key_local > q_local) sacc[kt][e] = masked;
          }
      }
      // tile max of the scaled logits (log2 units) over both half-rows
      float r;
      if (c2 > 0.f) {
        r = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) r = fmaxf(r, sacc[kt][e]);
        r = fmaxf(r, __shfl_xor(r, 32));
      } else {
        r = INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) r = fminf(r, sacc[kt][e]);
        r = fminf(r, __shfl_xor(r, 32));
      }
      const float m_tile = r * c2;
      const bool need = m_tile > m_used + kTau;
      if (__ballot(need)) {  // some query's max grew: move its reference
        const float m_new = need ? m_tile : m_used;
        const float alpha = sa::fast_exp2(m_used - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
        m_used = m_new;
      }
      // P = exp2(s c - m) packed to bf16 as the B operand of O^T += V^T P^T
      sa::u32x4 pb[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int e = 8 * h2 + 2 * w;
            pb[2 * kt + h2][w] = sa::pack_bf16x2(sa::fast_exp2(__builtin_fmaf(sacc[kt][e], c2, -m_used)),
                                                 sa::fast_exp2(__builtin_fmaf(sacc[kt][e + 1], c2, -m_used)));
          }
      // row sum over the rounded P actually fed to the MFMA
      float lsum = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) lsum = sa::dot2_bf16(pb[u][w], 0x3f803f80u, lsum);
      l_run += lsum;
      // O^T += V^T P^T; the V^T operand comes from transpose reads of row-major V
      const int gi = lane >> 4, ii = lane & 15;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int col = 32 * dt + 16 * (gi & 1) + 4 * (ii & 3);
        const int cs = col >> 3, half = (col >> 2) & 1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int keyA = 16 * u + 4 * hl + (ii >> 2);
          const int keyB = keyA + 8;
          const sa::u32x2 l2 = sa::lds_read_tr16(Vs + keyA * C::ROWB + swz_v(cs, keyA) * 16 + half * 8);
          const sa::u32x2 h2 = sa::lds_read_tr16(Vs + keyB * C::ROWB + swz_v(cs, keyB) * 16 + half * 8);
          const sa::u32x4 av = {l2[0], l2[1], h2[0], h2[1]};
          oacc[dt] = sa::mfma32(av, pb[u], oacc[dt]);
        }
      }
    }
  }

  // merge the groups' partial states into group 0
  l_run += __shfl_xor(l_run, 32);
  if constexpr (NP > 1) {
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the ring; reuse it
    float* mg = (float*)smem;
    constexpr int PER = D / 2 + 2;
    if (grp > 0) {
      float* slot = mg + (((grp - 1) * C::QW + wq) * 64 + lane) * PER;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) slot[16 * dt + e] = oacc[dt][e];
      slot[D / 2] = m_used;
      slot[D / 2 + 1] = l_run;
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < NP; ++g) {
      const float* slot = mg + (((g - 1) * C::QW + wq) * 64 + lane) * PER;
      const float mo = slot[D / 2], lo = slot[D / 2 + 1];
      const float mm = fmaxf(m_used, mo);
      const float ms = mm == -INFINITY ? 0.f : mm;
      const float a0 = sa::fast_exp2(m_used - ms), a1 = sa::fast_exp2(mo - ms);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = oacc[dt][e] * a0 + slot[16 * dt + e] * a1;
      l_run = l_run * a0 + lo * a1;
      m_used = mm;
    }
  }

  // normalise and store
  uint16_t* O = (uint16_t*)a.o + it.b * a.os[0] + it.h * a.os[1];
  float* L = a.lse + ((int64_t)it.b * a.H + it.h) * a.N;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
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
  if (hl == 0) L[qpos] = l_run > 0.f ? (m_used + log2f(l_run)) * sa::kLn2 : -INFINITY;
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
sa_status launch(Kern kern, const BsaArgs& a, int threads, int lds_bytes, hipStream_t stream,
                 const char* name) {
  const int64_t grid = (int64_t)a.B * a.H * a.nb;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), lds_bytes, stream, a);
  return sa_host::check_launch(name);
}

// (groups per workgroup NP, ring stages S) of each compiled tile shape
#ifndef SA_CFG_64_64
#define SA_CFG_64_64 1, 2
#endif
#ifndef SA_CFG_64_128
#define SA_CFG_64_128 1, 2
#endif
#ifndef SA_CFG_128_64
#define SA_CFG_128_64 1, 2
#endif
#ifndef SA_CFG_128_128
#define SA_CFG_128_128 1, 2
#endif

// The kernel must be named in a non-template context for its host stub to be
// emitted, hence a macro rather than a function template.
// Raise the dynamic-LDS limit of a kernel once (needed above 64 KiB).
inline sa_status allow_lds(const void* kern, int bytes) {
  if (bytes <= 65536) return SA_OK;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return e == hipSuccess ? SA_OK : sa_host::record_hip_error(e, "hipFuncSetAttribute");
}

#define SA_LAUNCH_BF16(D, BLK, CFG, NAME)                                                    \
  do {                                                                                       \
    using Cf = BsaCfg<D, BLK, CFG>;                                                          \
    static const sa_status lds_ok =                                                          \
        allow_lds((const void*)&bsa_fwd_bf16_kernel<D, BLK, CFG>, Cf::LDSB);                  \
    if (lds_ok != SA_OK) return lds_ok;                                                      \
    const int64_t grid = (int64_t)a.B * a.H * a.nb;                                          \
    hipLaunchKernelGGL((bsa_fwd_bf16_kernel<D, BLK, CFG>), dim3((unsigned)grid), dim3(Cf::NT), \
                       Cf::LDSB, stream, a);                                                 \
    return sa_host::check_launch(NAME);                                                      \
  } while (0)

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
  // A zero scale (uniform weights) is run as a tiny positive one: every logit
  // then rounds to 0 exactly as before, while masked logits still scale to -inf.
  a.scale_log2 = scale != 0.f ? scale * sa::kLog2e : 1e-30f;

  if (dtype == SA_BF16) {
    if (d == 64 && block == 64) SA_LAUNCH_BF16(64, 64, SA_CFG_64_64, "bsa_fwd_bf16<64,64>");
    if (d == 64 && block == 128) SA_LAUNCH_BF16(64, 128, SA_CFG_64_128, "bsa_fwd_bf16<64,128>");
    if (d == 128 && block == 64) SA_LAUNCH_BF16(128, 64, SA_CFG_128_64, "bsa_fwd_bf16<128,64>");
    SA_LAUNCH_BF16(128, 128, SA_CFG_128_128, "bsa_fwd_bf16<128,128>");
  }
  if (d == 64 && block == 64) return launch(bsa_fwd_f32_kernel<64, 64>, a, 64, 0, stream, "bsa_fwd_f32<64,64>");
  if (d == 64 && block == 128) return launch(bsa_fwd_f32_kernel<64, 128>, a, 128, 0, stream, "bsa_fwd_f32<64,128>");
  if (d == 128 && block == 64) return launch(bsa_fwd_f32_kernel<128, 64>, a, 64, 0, stream, "bsa_fwd_f32<128,64>");
  return launch(bsa_fwd_f32_kernel<128, 128>, a, 128, 0, stream, "bsa_fwd_f32<128,128>");
}
