// Token-level offset attention ("Depth-Staggered Fibonacci Spacing for Sparse
// Attention", Sec. 2, "Attended set"): query t attends the keys t - delta for
// every distance delta of a table shared by all queries (a dense window
// {0..W} plus rounded scaled Fibonacci rungs), skipping t - delta < 0.
//
// bf16 path (one workgroup = 4 waves walks consecutive 64-query tiles of one
// head; wave w owns queries t0 + 16 w + i, i < 16):
//   * near distances (<= 64): every key t - delta of the wave's 16 queries
//     lies in an 80-row band [t0 + 16 w - 64, t0 + 16 w + 16).  The band's
//     scores S^T = K Q^T and the product O^T += V^T P^T run on
//     v_mfma_f32_16x16x32_bf16 over the whole band; entries whose distance is
//     not in the table get weight 0 (a per-lane bit mask).  K / V rows reach
//     LDS by direct global->LDS copies into a ring of 64-row blocks: two when
//     a workgroup has one tile, three when it walks several (the next tile's
//     block is then in flight while the current one is used); each row is
//     copied once per workgroup.
//   * far rungs (> 64): each row is used by one query of the tile, so it is
//     gathered straight into registers (no LDS round trip), two rungs at a
//     time with an online-softmax rescale per batch; the K rows of batch b + 1
//     are in flight while the V rows of batch b are used.  The gather runs in
//     a layout of its own where the 4 lanes reading one row are adjacent
//     (lane 4 q + j: query q, 16-byte chunks 4 c + j), so each group of 4 lanes
//     reads one 64-byte segment; the MFMA layout has those lanes 16 apart,
//     which costs about 3x in L2 gather throughput.  The two layouts hold the
//     same (query, chunks) per lane up to the lane permutation 16 j + q <->
//     4 q + j, so q and the band's O^T state move across with ds_bpermute
//     once per tile; the O^T tiles take their rows in the permuted d order
//     that makes a lane's entries its gathered chunks.
//   * all global loads of the loop are issued as inline asm and waited for
//     with explicit vmcnt counts, so waiting for a far batch never waits for
//     the ring copies issued after it.
//   * workgroups of one head run on one XCD (blockIdx % 8 selects the XCD), so
//     the far-rung re-reads of a K / V row are served by its L2.
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
constexpr int kNearMax = 64;   // distances up to this are served by the MFMA band

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
  int32_t nnear;  // offsets[0 .. nnear) are <= kNearMax (bf16 path: MFMA band)
  int32_t near64; // 64 is a near distance
  uint64_t near_bits;  // bit x: distance x (< 64) is in the table
  int32_t tpw;    // 64-query tiles per workgroup (bf16 path)
  int32_t nchunk; // workgroups per (batch, head)
  float scale_log2;
  int32_t offs[SA_MAX_OFFSETS];
  int32_t nrung;  // interpolated rungs: key / value (1 - w) row[t - a] + w row[t - a - 1]
  int32_t rfloor[SA_MAX_RUNGS];
  float rw[SA_MAX_RUNGS];
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

// (v_a, v_b) bf16 pairs -> (lo halves), (hi halves)
__device__ __forceinline__ uint32_t pair_lo(uint32_t va, uint32_t vb) { return __builtin_amdgcn_perm(vb, va, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t va, uint32_t vb) { return __builtin_amdgcn_perm(vb, va, 0x07060302u); }

// 16-byte chunk slot of chunk c in a staged row: XOR with bits (0, 2, 1) of the
// row's low three bits, so that the 8 rows of one ds_read_b128 phase hit
// distinct slots and the 4 rows of one transpose-read phase fall in two
// different groups of four slots.
__device__ __forceinline__ int swz(int c, int row) {
  const int r = row & 7;
  return c ^ ((r & 1) | ((r & 2) << 1) | ((r & 4) >> 1));
}

// far rungs per register batch; resident workgroups per CU at d = 64; tiles
// per workgroup aim at this many workgroups per resident slot of the chip
// (each measured best against its neighbours)
constexpr int kFarBatch = 2;
constexpr int kWaves64 = 3;
constexpr int kTilesDiv = 4;

template <int D, int NS>
struct MCfg {
  static constexpr int NW = 4;               // waves per workgroup
  static constexpr int TQ = 64;              // queries per tile step (16 per wave)
  static constexpr int ROWB = 2 * D;         // bytes per K / V row
  static constexpr int RING = 64 * NS;       // staged rows: NS blocks of 64 rows
  static constexpr int RINGB = RING * ROWB;  // bytes of the K ring (the V ring follows)
  static constexpr int LDSB = 2 * RINGB;
  static constexpr int NC = D / 32;          // 16-byte chunks a lane holds per row
  static constexpr int NDT = D / 16;         // 16-row tiles of O^T
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;    // rows per copy wave-instruction
  static constexpr int IPW = ROWB / 64;      // copy wave-instructions per wave, block and matrix
  static constexpr int FC = kFarBatch;  // far rungs per register batch (even)
};

template <int D, int NS>
__global__ __launch_bounds__(256, D == 64 ? kWaves64 : 2) void offset_mfma_kernel(OffArgs a) {
  using C = MCfg<D, NS>;
  constexpr int NC = C::NC, NDT = C::NDT, FC = C::FC, ROWB = C::ROWB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t lds0 = sa::lds_addr(smem);

  const int lane = threadIdx.x & 63, w = sa::uniform(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int ntiles = (a.N + C::TQ - 1) / C::TQ;
  int bh, chunk;
  tile_of(blockIdx.x, a.B * a.H, a.nchunk, bh, chunk);
  const int ti0 = chunk * a.tpw, ti1 = min(ti0 + a.tpw, ntiles);
  const int b = bh / a.H, h = bh % a.H, kvh = h / (a.H / a.H_kv);

  const char* Qh = (const char*)((const uint16_t*)a.q + b * a.qs[0] + h * a.qs[1]);
  const char* Kh = (const char*)((const uint16_t*)a.k + b * a.ks[0] + kvh * a.ks[1]);
  const char* Vh = (const char*)((const uint16_t*)a.v + b * a.vs[0] + kvh * a.vs[1]);
  uint16_t* Oh = (uint16_t*)a.o + b * a.os[0] + h * a.os[1];
  float* Lh = a.lse + ((int64_t)b * a.H + h) * a.N;
  const uint32_t qrow = (uint32_t)a.qs[2] * 2u, krow = (uint32_t)a.ks[2] * 2u, vrow = (uint32_t)a.vs[2] * 2u;
  const bool has_near = a.nnear > 0;
  const int nfar = a.noff - a.nnear;
  const float c2 = a.scale_log2;

  // Band row of this lane's score (block kb, entry r): 16 kb + 4 g + r; its
  // distance from query i is 64 + i - (16 kb + 4 g + r).  nmask: the distance
  // is in the table; cmask: the key row is >= 0 in the first tile.
  uint32_t nmask = 0, cmask = 0;
#pragma unroll
  for (int kb = 0; kb < 5; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kb + 4 * g + r;
      const int dl = 64 + i - key;
      const bool in = dl >= 0 && dl <= 64 && (dl < 64 ? ((a.near_bits >> dl) & 1ull) != 0 : a.near64 != 0);
      nmask |= (uint32_t)in << (4 * kb + r);
      cmask |= (uint32_t)(key + 16 * w >= 64) << (4 * kb + r);
    }
  // LDS offsets inside a 16-row group: K operand (row i, chunk 4u + g) and the
  // transpose reads of V (row 4g + i/4, the 4 entries of O^T rows 4(i%4).. of
  // tile dt, i.e. d = 32(dt/2) + 8(i%4) + 4(dt%2) ..).
  uint32_t kofs[NC], vofs[NDT];
#pragma unroll
  for (int u = 0; u < NC; ++u) kofs[u] = i * ROWB + swz(4 * u + g, i) * 16;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int vr = 4 * g + (i >> 2);
    vofs[dt] = vr * ROWB + swz(4 * (dt >> 1) + (i & 3), vr) * 16 + 8 * (dt & 1);
  }

  // Copy 64-row block blk (>= -1) of K and V into ring slot blk mod 3.  Rows
  // outside [0, N) are clamped to a valid row: they only meet zero weights.
  // Every wave issues exactly 2 * IPW copies.
  auto stage = [&](int blk) {
    const uint32_t slot = (uint32_t)((blk + NS) % NS);
#pragma unroll
    for (int q = 0; q < C::IPW; ++q) {
      const int inst = q * C::NW + w;
      const int row = inst * C::RPI + lane / C::CPR;
      const int c = swz(lane % C::CPR, row);
      const int ar = min(max(blk * 64 + row, 0), a.N - 1);
      const uint32_t dst = lds0 + slot * (64 * ROWB) + inst * 1024;
      sa::dma16(Kh, (uint32_t)ar * krow + 16u * c, dst);
      sa::dma16(Vh, (uint32_t)ar * vrow + 16u * c, dst + C::RINGB);
    }
  };

  // Far-rung layout: lane 4 fq + fj holds query fq of the wave and chunks
  // 4 c + fj, so the 4 lanes that read one row are adjacent (one 64-byte
  // segment per group of 4 lanes).  It holds the same (query, chunks) as lane
  // 16 fj + fq of the MFMA layout: the two differ by a lane permutation.
  const int fq = lane >> 2, fj = lane & 3;
  const int to_far = (16 * fj + fq) * 4;  // bpermute address: MFMA layout -> far layout
  const int to_mfma = (4 * i) * 4;        // far layout -> MFMA layout (quad-uniform values)
  const uint32_t lone = fj == 0 ? 0x3f803f80u : 0u;  // far weights are counted once per query

  sa::u32x4 qb[NC], qf[NC];  // q in the MFMA layout (B operand) and in the far layout
  auto load_q = [&](int ti) {
    const int tq = min(ti * C::TQ + 16 * w + i, a.N - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) qb[c] = sa::gload16(Qh, (uint32_t)tq * qrow + 16u * (4 * c + g));
  };

  // Rows of far batch [n0, n0 + FC) of the far rungs from K or V (entries past
  // nfar repeat the last rung; their weight is 0): FC * NC loads.
  auto far_rows = [&](int n0, int tqf, const char* base, uint32_t rowb, sa::u32x4 (&buf)[FC][NC]) {
    uint32_t src[FC];
#pragma unroll
    for (int n = 0; n < FC; ++n) src[n] = (uint32_t)max(tqf - a.offs[a.nnear + min(n0 + n, nfar - 1)], 0);
#pragma unroll
    for (int n = 0; n < FC; ++n)
#pragma unroll
      for (int c = 0; c < NC; ++c) buf[n][c] = sa::gload16(base, src[n] * rowb + 16u * (4 * c + fj));
  };
  auto far_scores = [&](int n0, int tqf, sa::u32x4 (&kf)[FC][NC], float (&yf)[FC]) {
#pragma unroll
    for (int n = 0; n < FC; ++n) {
#pragma unroll
      for (int c = 0; c < NC; ++c) sa::tie(kf[n][c]);
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int x = 0; x < 4; ++x) dot = sa::dot2_bf16(qf[c][x], kf[n][c][x], dot);
      dot = sa::quad_sum(dot);
      const int dn = a.offs[a.nnear + min(n0 + n, nfar - 1)];
      const bool ok = (n0 + n < nfar) & (tqf >= dn);
      yf[n] = ok ? dot * c2 : -INFINITY;
    }
  };
  // O^T accumulators: MFMA layout during the band, far layout afterwards.
  // Entry [dt][r] is d = 8 (4 (dt/2) + lane chunk) + 4 (dt%2) + r.
  sa::f32x4 acc[NDT];
  float l = 0.f;
  // acc += pp.lo * row_a + pp.hi * row_b (bf16 pair weights), l += both weights
  auto pv_pair = [&](uint32_t pp, const sa::u32x4 (&va)[NC], const sa::u32x4 (&vb)[NC]) {
    l = sa::dot2_bf16(pp, lone, l);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        sa::f32x4& o = acc[2 * c + (x >> 1)];
        o[2 * (x & 1)] = sa::dot2_bf16(pp, pair_lo(va[c][x], vb[c][x]), o[2 * (x & 1)]);
        o[2 * (x & 1) + 1] = sa::dot2_bf16(pp, pair_hi(va[c][x], vb[c][x]), o[2 * (x & 1) + 1]);
      }
  };
  auto far_pv = [&](const float (&yf)[FC], float mu, sa::u32x4 (&vf)[FC][NC]) {
#pragma unroll
    for (int n = 0; n < FC; ++n)
#pragma unroll
      for (int c = 0; c < NC; ++c) sa::tie(vf[n][c]);
#pragma unroll
    for (int n = 0; n < FC; n += 2)
      pv_pair(sa::pack_bf16x2(sa::fast_exp2(yf[n] - mu), sa::fast_exp2(yf[n + 1] - mu)), vf[n], vf[n + 1]);
  };
  // rescale the running state to a new maximum mb > m
  auto rescale = [&](float& m, float mb) {
    const float alpha = sa::fast_exp2(m - mb);
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[dt][r] *= alpha;
    m = mb;
  };

  if (has_near) {
    stage(ti0 - 1);
    stage(ti0);
  }
  load_q(ti0);

  for (int ti = ti0; ti < ti1; ++ti) {
    sa::vm_wait<0>();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      sa::tie(qb[c]);
#pragma unroll
      for (int x = 0; x < 4; ++x) qf[c][x] = __float_as_uint(sa::bperm(to_far, __uint_as_float(qb[c][x])));
    }
    __syncthreads();  // ring blocks ti - 1, ti are in LDS; block ti - 2 is free
    const int t0 = ti * C::TQ;
    const int tf = t0 + 16 * w + fq, tqf = min(tf, a.N - 1);
    const bool dma = NS == 3 && has_near && ti + 1 < ti1;

    sa::u32x4 kf[FC][NC], vf[FC][NC];
    if (nfar > 0) {
      far_rows(0, tqf, Kh, krow, kf);
      far_rows(0, tqf, Vh, vrow, vf);
    }
    if (dma) stage(ti + 1);

#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = sa::f32x4{0.f, 0.f, 0.f, 0.f};
    l = 0.f;
    float y[20];
    float mx = -INFINITY;  // MFMA layout, per query
    // ring row of band row 0 (the band starts at t0 + 16 w - 64)
    const int rb = (t0 + 16 * w + C::RING - 64) % C::RING;
    if (has_near) {
#pragma unroll
      for (int kb = 0; kb < 5; ++kb) {
        int rr = rb + 16 * kb;
        rr = rr >= C::RING ? rr - C::RING : rr;
        sa::f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NC; ++u) {
          const sa::u32x4 kv = *(const sa::u32x4*)(smem + rr * ROWB + kofs[u]);
          s = sa::mfma16(kv, qb[u], s);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) y[4 * kb + r] = s[r] * c2;
      }
      const uint32_t vm = t0 == 0 ? (nmask & cmask) : nmask;
#pragma unroll
      for (int e = 0; e < 20; ++e) {
        y[e] = ((vm >> e) & 1u) ? y[e] : -INFINITY;
        mx = fmaxf(mx, y[e]);
      }
      mx = sa::max_xor32(sa::max_xor16(mx));
    }
    float yf[FC];
    if (nfar > 0) {
      if (dma)
        sa::vm_wait<FC * NC + 2 * C::IPW>();
      else
        sa::vm_wait<FC * NC>();
      far_scores(0, tqf, kf, yf);
      float mf = yf[0];
#pragma unroll
      for (int n = 1; n < FC; ++n) mf = fmaxf(mf, yf[n]);
      mx = fmaxf(mx, sa::bperm(to_mfma, mf));
    }
    // running max, the same value in both layouts
    float m = sa::bperm(to_far, mx);
    float mu = m == -INFINITY ? 0.f : m;
    if (has_near) {
      const float muc = mx == -INFINITY ? 0.f : mx;
      uint32_t pk[5][2];
      float ln = 0.f;
#pragma unroll
      for (int kb = 0; kb < 5; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          pk[kb][j] = sa::pack_bf16x2(sa::fast_exp2(y[4 * kb + 2 * j] - muc), sa::fast_exp2(y[4 * kb + 2 * j + 1] - muc));
          ln = sa::dot2_bf16(pk[kb][j], 0x3f803f80u, ln);
        }
#pragma unroll
      for (int st = 0; st < 3; ++st) {
        int r0 = rb + 32 * st;
        r0 = r0 >= C::RING ? r0 - C::RING : r0;
        int r1 = r0 + 16;
        r1 = r1 >= C::RING ? r1 - C::RING : r1;
        const sa::u32x4 bop = {pk[2 * st][0], pk[2 * st][1], st < 2 ? pk[2 * st + 1][0] : 0u,
                               st < 2 ? pk[2 * st + 1][1] : 0u};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const sa::u32x2 v0 = sa::lds_read_tr16(smem + C::RINGB + r0 * ROWB + vofs[dt]);
          sa::u32x2 v1 = {0u, 0u};
          if (st < 2) v1 = sa::lds_read_tr16(smem + C::RINGB + r1 * ROWB + vofs[dt]);
          acc[dt] = sa::mfma16(sa::u32x4{v0[0], v0[1], v1[0], v1[1]}, bop, acc[dt]);
        }
      }
      // band state -> far layout
      ln = sa::sum_xor32(sa::sum_xor16(ln));
      l = sa::bperm(to_far, ln);
      l = fj == 0 ? l : 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][r] = sa::bperm(to_far, acc[dt][r]);
    }
    // Far batches, software-pipelined by one half: K of batch b + 1 is in
    // flight while V of batch b is used, and V of batch b + 1 while the scores
    // of batch b + 1 are formed (queue order: K0 V0 [copies] K1 V1 K2 ...).
    if (nfar > 0) {
      for (int n0 = 0; n0 < nfar; n0 += FC) {
        const bool more = n0 + FC < nfar;
        if (more) far_rows(n0 + FC, tqf, Kh, krow, kf);
        if (n0 == 0 && dma) {
          if (more)
            sa::vm_wait<2 * C::IPW + FC * NC>();
          else
            sa::vm_wait<2 * C::IPW>();
        } else {
          if (more)
            sa::vm_wait<FC * NC>();
          else
            sa::vm_wait<0>();
        }
        far_pv(yf, mu, vf);
        if (!more) break;
        far_rows(n0 + FC, tqf, Vh, vrow, vf);
        sa::vm_wait<FC * NC>();
        far_scores(n0 + FC, tqf, kf, yf);
        float mb = yf[0];
#pragma unroll
        for (int n = 1; n < FC; ++n) mb = fmaxf(mb, yf[n]);
        if (mb > m) rescale(m, mb);  // per query (its 4 lanes agree)
        mu = m == -INFINITY ? 0.f : m;
      }
    }
    // Interpolated rungs, one online-softmax step each: rows t - a and
    // t - a - 1 (both exist for t >= a + 1); the score is the same blend of
    // the two rows' dot products, and the weight p splits into p (1 - w) and
    // p w over the two value rows.
    for (int r = 0; r < a.nrung; ++r) {
      const int ra = a.rfloor[r];
      const float rwt = a.rw[r];
      const uint32_t s0 = (uint32_t)max(tqf - ra, 0), s1 = (uint32_t)max(tqf - ra - 1, 0);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        kf[0][c] = sa::gload16(Kh, s0 * krow + 16u * (4 * c + fj));
        kf[1][c] = sa::gload16(Kh, s1 * krow + 16u * (4 * c + fj));
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        vf[0][c] = sa::gload16(Vh, s0 * vrow + 16u * (4 * c + fj));
        vf[1][c] = sa::gload16(Vh, s1 * vrow + 16u * (4 * c + fj));
      }
      sa::vm_wait<2 * NC>();
      float dot[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
#pragma unroll
        for (int c = 0; c < NC; ++c) sa::tie(kf[n][c]);
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) x = sa::dot2_bf16(qf[c][e], kf[n][c][e], x);
        dot[n] = sa::quad_sum(x);
      }
      const float y = tqf >= ra + 1 ? ((1.f - rwt) * dot[0] + rwt * dot[1]) * c2 : -INFINITY;
      if (y > m) rescale(m, y);
      const float p = sa::fast_exp2(y - (m == -INFINITY ? 0.f : m));
      sa::vm_wait<0>();
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int c = 0; c < NC; ++c) sa::tie(vf[n][c]);
      pv_pair(sa::pack_bf16x2(p * (1.f - rwt), p * rwt), vf[0], vf[1]);
    }

    l = sa::quad_sum(l);
    if (tf < a.N) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* orow = Oh + (int64_t)tf * a.os[2];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const sa::f32x4& o0 = acc[2 * c];
        const sa::f32x4& o1 = acc[2 * c + 1];
        const sa::u32x4 wv = {sa::pack_bf16x2(o0[0] * inv, o0[1] * inv), sa::pack_bf16x2(o0[2] * inv, o0[3] * inv),
                              sa::pack_bf16x2(o1[0] * inv, o1[1] * inv), sa::pack_bf16x2(o1[2] * inv, o1[3] * inv)};
        *(sa::u32x4*)(orow + 8 * (4 * c + fj)) = wv;
      }
      if (fj == 0) Lh[tf] = l > 0.f ? (m + log2f(l)) * sa::kLn2 : -INFINITY;
    }
    if (ti + 1 < ti1) load_q(ti + 1);
  }
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

  // interpolated rungs (valid for t >= a + 1), one rescale step each
  for (int r = 0; r < a.nrung; ++r) {
    const int ra = a.rfloor[r];
    if (t < ra + 1) continue;
    const float w = a.rw[r];
    float k0[D], k1[D];
    load_row<D, BF16>(K + (int64_t)(t - ra) * a.ks[2], k0);
    load_row<D, BF16>(K + (int64_t)(t - ra - 1) * a.ks[2], k1);
    float dot = 0.f;
#pragma unroll
    for (int x = 0; x < D; ++x) dot = fmaf(qf[x], fmaf(w, k1[x] - k0[x], k0[x]), dot);
    const float y = dot * c2;
    const float m_new = fmaxf(m, y);
    const float alpha = sa::fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int x = 0; x < D; ++x) acc[x] *= alpha;
    m = m_new;
    const float p = sa::fast_exp2(y - m);
    l += p;
    load_row<D, BF16>(V + (int64_t)(t - ra) * a.vs[2], k0);
    load_row<D, BF16>(V + (int64_t)(t - ra - 1) * a.vs[2], k1);
#pragma unroll
    for (int x = 0; x < D; ++x) acc[x] = fmaf(p, fmaf(w, k1[x] - k0[x], k0[x]), acc[x]);
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

template <int D, int NS>
sa_status launch_mfma(const OffArgs& a, dim3 grid, hipStream_t stream) {
  using Cf = MCfg<D, NS>;
  static const sa_status lds_ok = allow_lds((const void*)&offset_mfma_kernel<D, NS>, Cf::LDSB);
  if (lds_ok != SA_OK) return lds_ok;
  hipLaunchKernelGGL((offset_mfma_kernel<D, NS>), grid, dim3(256), Cf::LDSB, stream, a);
  return SA_OK;
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

extern "C" sa_status offset_attn_make_table_ratio(int32_t W, int64_t num, int64_t den, const int64_t* base,
                                                  int32_t K, int32_t N, int32_t* table_out, int32_t capacity,
                                                  int32_t* count_out) {
  if (!table_out || !count_out || (K > 0 && !base)) return SA_ERR_NULL;
  if (W < 0 || K < 0 || N < 1 || capacity < 0) return SA_ERR_INVALID;
  const int64_t lim = (int64_t)1 << 31;
  if (num < 0 || num >= lim || den < 1 || den >= lim) return SA_ERR_INVALID;
  std::vector<int64_t> d;
  for (int64_t x = 0; x <= W && x < N; ++x) d.push_back(x);
  for (int j = 0; j < K; ++j) {
    if (base[j] < 0 || base[j] >= lim) return SA_ERR_INVALID;
    const int64_t x = (2 * num * base[j] + den) / (2 * den);  // floor(num f / den + 1/2), f >= 0
    if (x < N) d.push_back(x);
  }
  std::sort(d.begin(), d.end());
  d.erase(std::unique(d.begin(), d.end()), d.end());
  if ((int64_t)d.size() > capacity) return SA_ERR_CAPACITY;
  for (size_t j = 0; j < d.size(); ++j) table_out[j] = (int32_t)d[j];
  *count_out = (int32_t)d.size();
  return SA_OK;
}

extern "C" sa_status offset_attn_make_interp(int32_t W, double alpha, const int64_t* base, int32_t K, int32_t N,
                                             int32_t* table_out, int32_t capacity, int32_t* count_out,
                                             int32_t* rung_floor, float* rung_weight, int32_t rung_capacity,
                                             int32_t* rung_count) {
#pragma clang fp contract(off)
  if (!table_out || !count_out || !rung_floor || !rung_weight || !rung_count || (K > 0 && !base))
    return SA_ERR_NULL;
  if (W < 0 || K < 0 || N < 1 || capacity < 0 || rung_capacity < 0 || !isfinite(alpha)) return SA_ERR_INVALID;
  std::vector<int64_t> d;
  std::vector<std::pair<int32_t, float>> rungs;
  for (int64_t x = 0; x <= W && x < N; ++x) d.push_back(x);
  for (int j = 0; j < K; ++j) {
    if (base[j] < 0) return SA_ERR_INVALID;
    const double x = alpha * (double)base[j];
    if (x < 0.0) continue;  // negative distances reach no key
    const double fl = floor(x);
    if (x == fl) {
      if (x < (double)N) d.push_back((int64_t)x);
    } else if (fl + 1.0 <= (double)N - 1.0) {
      rungs.push_back({(int32_t)fl, (float)(x - fl)});
    }
  }
  std::sort(d.begin(), d.end());
  d.erase(std::unique(d.begin(), d.end()), d.end());
  if ((int64_t)d.size() > capacity || (int64_t)rungs.size() > rung_capacity) return SA_ERR_CAPACITY;
  for (size_t j = 0; j < d.size(); ++j) table_out[j] = (int32_t)d[j];
  for (size_t r = 0; r < rungs.size(); ++r) rung_floor[r] = rungs[r].first, rung_weight[r] = rungs[r].second;
  *count_out = (int32_t)d.size();
  *rung_count = (int32_t)rungs.size();
  return SA_OK;
}

// Shared by both offset entry points (nrung = 0: integer distances only).
static sa_status offset_run(int32_t dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                            int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d, const int64_t* strides,
                            const int32_t* offsets, int32_t num_offsets, const int32_t* rung_floor,
                            const float* rung_weight, int32_t num_rungs, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || (num_offsets > 0 && !offsets)) return SA_ERR_NULL;
  if (num_rungs > 0 && (!rung_floor || !rung_weight)) return SA_ERR_NULL;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_INVALID;
  if (B < 1 || H < 1 || H_kv < 1 || N < 1 || d < 1) return SA_ERR_INVALID;
  if (H % H_kv != 0) return SA_ERR_INVALID;
  if (!isfinite(scale)) return SA_ERR_INVALID;
  if (num_offsets < 0 || num_offsets > SA_MAX_OFFSETS) return SA_ERR_INVALID;
  if (num_rungs < 0 || num_rungs > SA_MAX_RUNGS || num_offsets + num_rungs < 1) return SA_ERR_INVALID;
  for (int n = 0; n < num_offsets; ++n) {
    if (offsets[n] < 0 || offsets[n] >= N) return SA_ERR_INVALID;
    if (n > 0 && offsets[n] <= offsets[n - 1]) return SA_ERR_INVALID;
  }
  for (int r = 0; r < num_rungs; ++r) {
    if (rung_floor[r] < 0 || (int64_t)rung_floor[r] + 1 > (int64_t)N - 1) return SA_ERR_INVALID;
    if (!(rung_weight[r] >= 0.f && rung_weight[r] <= 1.f)) return SA_ERR_INVALID;
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
  a.nrung = num_rungs;
  for (int r = 0; r < num_rungs; ++r) a.rfloor[r] = rung_floor[r], a.rw[r] = rung_weight[r];
  a.nnear = 0;
  a.near_bits = 0;
  a.near64 = 0;
  while (a.nnear < num_offsets && offsets[a.nnear] <= kNearMax) {
    const int x = offsets[a.nnear++];
    if (x < 64)
      a.near_bits |= 1ull << x;
    else
      a.near64 = 1;
  }
  if (dtype == SA_BF16) {
    // rows are addressed with 32-bit byte offsets from the head's base
    const int64_t rowb = std::max(st[0].s, std::max(st[1].s, st[2].s)) * 2;
    if ((int64_t)N * rowb > 0xffffffffll) return SA_ERR_UNSUPPORTED;
    // tiles per workgroup: keep at least ~4 workgroups per slot of the chip
    // (256 CUs x 3 resident workgroups); a longer walk re-copies fewer halo rows
    const int64_t ntiles = ((int64_t)N + 63) / 64;
    const int64_t total = (int64_t)B * H * ntiles;
    a.tpw = (int32_t)std::max<int64_t>(1, std::min<int64_t>(ntiles, total / (kTilesDiv * 256 * 3)));
    a.nchunk = (int32_t)((ntiles + a.tpw - 1) / a.tpw);
    if ((int64_t)B * H * a.nchunk > 0x7fffffffll) return SA_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((int64_t)B * H * a.nchunk));
    // two ring slots when every workgroup has one tile (no block is prefetched)
    sa_status ls;
    if (d == 64)
      ls = a.tpw == 1 ? launch_mfma<64, 2>(a, grid, stream) : launch_mfma<64, 3>(a, grid, stream);
    else
      ls = a.tpw == 1 ? launch_mfma<128, 2>(a, grid, stream) : launch_mfma<128, 3>(a, grid, stream);
    if (ls != SA_OK) return ls;
  } else {
    const dim3 grid((unsigned)((int64_t)B * H * tiles));
    if (d == 64)
      hipLaunchKernelGGL((offset_fwd_kernel<64, false>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((offset_fwd_kernel<128, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return sa_host::check_launch("offset_fwd_kernel");
}

extern "C" sa_status offset_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                                     void* o, float* lse, int32_t B, int32_t H, int32_t H_kv,
                                     int32_t N, int32_t d, const int64_t* strides,
                                     const int32_t* offsets, int32_t num_offsets, float scale,
                                     hipStream_t stream) {
  if (!offsets) return SA_ERR_NULL;
  if (num_offsets < 1) return SA_ERR_INVALID;
  return offset_run(dtype, q, k, v, o, lse, B, H, H_kv, N, d, strides, offsets, num_offsets, nullptr,
                    nullptr, 0, scale, stream);
}

extern "C" sa_status offset_attn_fwd_interp(int32_t dtype, const void* q, const void* k, const void* v,
                                            void* o, float* lse, int32_t B, int32_t H, int32_t H_kv,
                                            int32_t N, int32_t d, const int64_t* strides,
                                            const int32_t* offsets, int32_t num_offsets,
                                            const int32_t* rung_floor, const float* rung_weight,
                                            int32_t num_rungs, float scale, hipStream_t stream) {
  return offset_run(dtype, q, k, v, o, lse, B, H, H_kv, N, d, strides, offsets, num_offsets, rung_floor,
                    rung_weight, num_rungs, scale, stream);
}
