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
//     optionally NP groups of waves split the row's key tiles and merge;
//   * key blocks are walked in 64-key tiles copied global -> LDS by direct
//     (DMA) loads into K and V slots: one slot each for whole rows (small LDS
//     footprint, many resident workgroups), a ring for split rows at d = 64
//     whose K side runs one tile ahead so that S(n+1) is computed on the
//     matrix cores while the softmax of tile n runs on the VALU;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16, so every lane owns one query
//     column: the row max / sum of the online softmax are in-lane except for a
//     single exchange with lane ^ 32 (v_permlane32_swap);
//   * O^T += V^T P^T on the same MFMA: the fp32 accumulator of S^T already holds
//     exactly the keys each lane must supply as the P operand, so P goes from
//     the accumulator to the operand registers with one bf16 pack and no LDS
//     round trip.  The V^T operand comes from row-major V in LDS through
//     transpose reads (ds_read_b64_tr_b16);
//   * in the one-slot kernels the K and V^T operand reads of a step are issued
//     in a fixed order a few MFMAs ahead of their use (scheduling barriers
//     hold that order; the compiler's own waits count them), instead of each
//     MFMA waiting out a full LDS round trip;
//   * 16-byte LDS chunks are XOR-swizzled so that the K operand reads
//     (ds_read_b128, sa::lds_slot) and the V^T transpose reads
//     (sa::lds_slot_tr) are free of bank conflicts on gfx950's 64-bank LDS;
//   * launch order follows `sched` (longest rows first); blockIdx % (B*H) picks
//     the head, so with B*H a multiple of 8 every query block of one head runs
//     on the same XCD and shares its L2.
// fp32 path: a plain VALU kernel, one thread per query, for exact checks.
#include <math.h>

#include <mutex>
#include <type_traits>

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
  float scale_log2;  // |scale| * log2(e) (bf16 path), never 0
  uint32_t qsign;    // bf16 pair sign mask folded into Q when scale < 0
  // Split rows (whole-row kernels only): the first split_rows launch positions
  // of every head are each run by split_ways workgroups, part p taking tiles
  // p, p + split_ways, ...; their partial softmax states meet in the workspace.
  int32_t split_rows, split_ways;
  int32_t* split_cnt;  // arrival counter of split row bh * split_rows + pos, 0 between launches
  float* split_part;   // [B * H * split_rows][split_ways] partial states
};

// Work item of a workgroup: head (b, h), query block i, CSR entry range.
struct Item {
  int32_t b, h, kvh, i;
  int32_t e_beg, e_end;
  bool ok;
};

// Work item of head bh = b * H + h at launch position pos of its mask group.
__device__ __forceinline__ Item work_item_at(const BsaArgs& a, int32_t bh, int32_t pos) {
  Item it;
  it.b = bh / a.H;
  it.h = bh - it.b * a.H;
  it.kvh = it.h / (a.H / a.H_kv);
  const int64_t g = (int64_t)it.b * a.mbs + (int64_t)it.h * a.mhs;
  it.i = sa::uniform(a.sched ? a.sched[g * a.nb + pos] : pos);
  it.ok = it.i >= 0 && it.i < a.nb;
  const int64_t r = g * a.nb + (it.ok ? it.i : 0);
  int64_t e0 = a.row_ptr[r], e1 = a.row_ptr[r + 1];
  e0 = max((int64_t)0, min(e0, a.col_capacity));
  e1 = max(e0, min(e1, a.col_capacity));
  // row_ptr entries are int32, so the clamped range fits in 32 bits; the
  // values are the same in every lane (made visible to the compiler)
  it.e_beg = sa::uniform((int32_t)e0);
  it.e_end = sa::uniform((int32_t)e1);
  return it;
}

// One row per workgroup: blockIdx = pos * (B * H) + bh.
__device__ __forceinline__ Item work_item(const BsaArgs& a) {
  const int32_t BH = a.B * a.H;
  const int32_t pos = blockIdx.x / BH;
  return work_item_at(a, blockIdx.x - pos * BH, pos);
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
// at the end.
//
// K and V travel global -> LDS by direct (DMA) loads into two rings of S
// slots.  Two shapes of the tile loop:
//   * one slot (S = 1, not pipelined; the row_split = 1 configurations): step n
//     computes S(n), the softmax and O += V(n) P(n), then, after a barrier,
//     copies tile n+1 into the slots.  The copy latency of a tile is covered by
//     the other resident workgroups rather than by a deeper ring: with 16 KiB
//     of LDS per workgroup (d = 64) occupancy is set by registers alone, four
//     waves per SIMD at d = 64 (three at d = 128), which measured faster than
//     two slots with fewer resident workgroups;
//   * pipelined (PIPE, S >= 2; the d = 64 split-row configurations): while the
//     softmax of tile n runs on the VALU, the MFMAs of S(n+1) = K(n+1) Q^T are
//     already in flight, and the MFMAs of O += V(n) P(n) overlap the
//     bookkeeping of the next step; the K ring runs one tile ahead of the V
//     ring, so at step n the slots of K(n+1) and V(n) are read while K(n+S) and
//     V(n+S-1) are in flight.
// The row's key-block ids are held in VGPR lanes and read with v_readlane, so
// the loop issues no memory access besides the DMA and LDS operand reads.

// Workgroup barrier that does not drain outstanding DMA loads (a fenced
// barrier would wait for every in-flight tile, not just the one needed).
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most c * J vector loads of this wave are outstanding (c <= 4).
template <int J>
__device__ __forceinline__ void wait_vm_units(int c) {
  switch (c) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<J>(); break;
    case 2: wait_vmcnt<2 * J>(); break;
    case 3: wait_vmcnt<3 * J>(); break;
    default: wait_vmcnt<4 * J>(); break;
  }
}


// Software-pipeline shape: K operand k-steps read ahead, VALU instructions
// scheduled after each S(n+1) MFMA.
constexpr int kKPre = 4;
constexpr int kVGroup = 12;
// One-slot kernels: K operands read this many MFMAs ahead of their use, V
// operands put in flight before the softmax of a tile and this many ahead
// during O += V P (deeper rings spill at d = 128).
constexpr int kKAhead = 3;
constexpr int kVAhead = 2;
constexpr int kVRing = 3;

template <int D, int BLK, int NP, int S, bool PIPE>
struct BsaCfg {
  static constexpr int QW = BLK / 32;          // waves per group
  static constexpr int NW = QW * NP;           // waves per workgroup
  static constexpr int NT = NW * 64;           // threads
  static constexpr int SUBS = BLK / 64;        // 64-key tiles per key block
  static constexpr int CPR = D / 8;            // 16-byte chunks per K / V row
  static constexpr int ROWB = D * 2;           // bytes per K / V row
  static constexpr int KVB = 64 * ROWB;        // bytes of one K (or V) tile
  static constexpr int SLOTB = NP * KVB;       // one ring slot: a tile per group
  static constexpr int VRING = S * SLOTB;      // offset of the V ring
  static constexpr int RINGB = 2 * S * SLOTB;
  static constexpr int JN = KVB / 16 / (QW * 64);  // DMA loads per thread per tile
  // K operand k-steps of the next tile read at the top of a step (the rest
  // are read inside the MFMA / softmax interleave)
  static constexpr int KPRE = kKPre < D / 16 ? kKPre : D / 16;
  static constexpr int KPA = KPRE > 0 ? KPRE : 1;
  static_assert(S >= 1 && S <= 3 && (S >= 2 || !PIPE), "1 to 3 ring slots, at least 2 when pipelined");
  static_assert(JN >= 1 && (KVB / 16) % (QW * 64) == 0, "tiles must split evenly over a group");
  static_assert(4 * JN < 64, "vmcnt range");
  // merge area: per (group > 0, wave, lane): O^T partial (D/2 floats), m, l
  static constexpr int MERGEB = (NP - 1) * QW * 64 * (D / 2 + 2) * 4;
  static constexpr int LDSB = RINGB > MERGEB ? RINGB : MERGEB;  // dynamic LDS bytes
};

template <int D, int BLK, int NP, int S, bool PIPE>
// Whole-row kernels keep the register count of 4 (d = 64) or 3 (d = 128) waves
// per SIMD.
__global__ __launch_bounds__(BLK / 32 * NP * 64)
__attribute__((amdgpu_waves_per_eu(NP == 1 && !PIPE ? (D == 128 ? 3 : 4) : 1)))
void bsa_fwd_bf16_kernel(BsaArgs a) {
  using C = BsaCfg<D, BLK, NP, S, PIPE>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = sa::uniform(tid >> 6);
  const int grp = wave / C::QW, wq = wave % C::QW;
  const int hl = lane >> 5, lq = lane & 31;

  // Work unit: a whole row, or one part of a split row (whole-row kernels):
  // per head, units W p .. W p + W - 1 are the parts of the row at launch
  // position p < split_rows (W = split_ways), unit u >= W split_rows the row at
  // u - (W - 1) split_rows.
  Item it;
  int part = -1;  // >= 0: this workgroup takes tiles part, part + W, ... of the row
  int32_t unit_bh = 0, unit_pos = 0;
  if (NP == 1 && a.split_rows > 0) {
    const int32_t BH = a.B * a.H, W = a.split_ways;
    const int32_t u = blockIdx.x / BH;
    unit_bh = blockIdx.x - u * BH;
    if (u < W * a.split_rows) {
      unit_pos = u / W;
      part = u - unit_pos * W;
    } else {
      unit_pos = u - (W - 1) * a.split_rows;
    }
    it = work_item_at(a, unit_bh, unit_pos);
  } else {
    it = work_item(a);
  }
  if (!it.ok) return;
  const int np = part >= 0 ? a.split_ways : NP;  // tile stride of this group
  const int gs = part >= 0 ? part : grp;         // ... and its first tile

  const uint16_t* Q = (const uint16_t*)a.q + it.b * a.qs[0] + it.h * a.qs[1];
  const uint16_t* K = (const uint16_t*)a.k + it.b * a.ks[0] + it.kvh * a.ks[1];
  const uint16_t* V = (const uint16_t*)a.v + it.b * a.vs[0] + it.kvh * a.vs[1];
  const int64_t ks2 = a.ks[2], vs2 = a.vs[2];
  const int32_t limit = a.causal ? it.i + 1 : a.nb;  // usable key blocks are < limit

  // Q^T as the B operand: lane holds query lq of this wave, d = 16 k + 8 hl .. +7.
  // A negative scale is folded into Q (exact sign flip), so the softmax below
  // always works with a positive log2 scale.
  const int q_local = wq * 32 + lq;
  const int64_t qpos = (int64_t)it.i * BLK + q_local;
  sa::u32x4 qr[D / 16];
#pragma unroll
  for (int k = 0; k < D / 16; ++k) {
    qr[k] = *(const sa::u32x4*)(Q + qpos * a.qs[2] + 16 * k + 8 * hl);
#pragma unroll
    for (int w = 0; w < 4; ++w) qr[k][w] ^= a.qsign;
  }

  sa::f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  // Running reference max (log2 units).  Finite start: a fully masked tile
  // then yields exp2(-inf) = 0 instead of inf - inf.
  float m_used = -1e30f;
  const float c2 = a.scale_log2;  // > 0
  constexpr float kTau = 8.f;     // rescale only when the running max grows by > 2^8

  // DMA plan: copy j of wave wq of a group moves chunks [64 (j QW + wq), +64)
  // of the group's K (or V) tile, i.e. whole rows (RPC rows per copy); lane i
  // lands at 16 i past the copy's LDS base and reads the global chunk that
  // belongs in that slot (sa::lds_slot is its own inverse).  Copy j reads rows
  // RPC j further down than copy 0; when RPC is a multiple of the slot
  // pattern's period one per-lane source offset serves every copy, otherwise
  // (RPC = 8: d = 128 with 64-query blocks) odd copies take a second one.
  // When the rows of a tile are contiguous in global memory (sequence stride =
  // d) and copies j, j + 1 are 2048 bytes apart in both spaces with one
  // offset, they share one M0 setup.
  constexpr int RPC = C::QW * 64 / C::CPR;  // rows per copy
  static_assert(RPC % 8 == 0, "copies hold whole rows");
  constexpr bool kOddSlots = RPC % sa::kSlotPeriod != 0;
  uint32_t offK, offV, offK1, offV1;
  {
    const int r = wq * 64 + lane;  // chunk of this lane in copy 0
    const int key = r / C::CPR, cs = r % C::CPR;
    offK = (uint32_t)(key * ks2 * 2) + 16u * (uint32_t)sa::lds_slot<D>(cs, key);
    offV = (uint32_t)(key * vs2 * 2) + 16u * (uint32_t)sa::lds_slot_tr<D>(cs, key);
    offK1 = kOddSlots ? (uint32_t)(key * ks2 * 2) + 16u * (uint32_t)sa::lds_slot<D>(cs, key + RPC) : offK;
    offV1 = offV;  // the V pattern repeats every 4 rows
  }
  constexpr bool kPairs = C::QW * 64 * 16 == 2048 && C::JN % 4 == 0 && !kOddSlots;
  const bool k_contig = kPairs && ks2 == D, v_contig = kPairs && vs2 == D;
  const uint32_t kring = sa::lds_addr(smem) + grp * C::KVB;
  const uint32_t vring = kring + C::VRING;
  const uint8_t* const kring_p = smem + grp * C::KVB;
  const uint8_t* const vring_p = kring_p + C::VRING;
  // One-slot kernels read the MFMA operands in a fixed order, a few MFMAs
  // ahead of their use.  K operand of k-step k for the lane's key lq (keys
  // 32 kt + lq sit 32 rows further, the same slot pattern); V^T operand of the
  // lane's d-column group dt for keys 4 hl + (lane & 15) / 4 (16 u + 8 more
  // rows down share the pattern, period 4).
  constexpr bool kHand = !PIPE && S == 1;
  const uint8_t* kop_p[D / 16];
  const uint8_t* vop_p[D / 32];
  if constexpr (kHand) {
#pragma unroll
    for (int k = 0; k < D / 16; ++k) kop_p[k] = kring_p + lq * C::ROWB + 16 * sa::lds_slot<D>(2 * k + hl, lq);
    const int gi = lane >> 4, ii = lane & 15;
    const int key0 = 4 * hl + (ii >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int col = 32 * dt + 16 * (gi & 1) + 4 * (ii & 3);
      vop_p[dt] = vring_p + key0 * C::ROWB + 16 * sa::lds_slot_tr<D>(col >> 3, key0) + 8 * ((col >> 2) & 1);
    }
  }

  // Copies of one 64-key tile (key block kb >= 0, sub-tile sub) into a ring
  // slot.  Byte offsets of a block are below 2^32 (the host bounds the
  // sequence strides), so a 32 x 32-bit product locates the tile.
  const uint32_t kbs = (uint32_t)(BLK * ks2 * 2), vbs = (uint32_t)(BLK * vs2 * 2);  // bytes per key block
  const uint32_t offK4 = offK + 4096u, offV4 = offV + 4096u;
  auto dma_tile = [&](const uint16_t* X, uint32_t xbs, int64_t xs2, uint32_t off, uint32_t off1, uint32_t off4,
                      bool contig, uint32_t ring, int slot, int32_t kb, int sub) {
    const char* src = (const char*)X + (uint64_t)(uint32_t)kb * xbs + (uint32_t)(sub * 64 * xs2 * 2);
    const uint32_t dst = ring + slot * C::SLOTB + wq * 64 * 16;
    if (contig) {  // pairs 2048 bytes apart, two pairs per M0 save
#pragma unroll
      for (int j = 0; j < C::JN; j += 4) sa::dma16x4p(src + j * 2048, off, off4, dst + j * 2048);
    } else {
#pragma unroll
      for (int j = 0; j < C::JN; ++j)
        sa::dma16(src + (uint64_t)j * RPC * xs2 * 2, (j & 1) ? off1 : off, dst + j * C::QW * 64 * 16);
    }
  };

  sa::f32x16 sA[2], sB[2];
  float ls[4] = {0.f, 0.f, 0.f, 0.f};  // partial row sums (l = their total)
  bool first_pass = true;
  for (int64_t base = it.e_beg; base < it.e_end; base += 64) {
    const int cnt = (int)min((int64_t)64, it.e_end - base);
    // key-block ids of the pass, entry x in lane x
    const int lst = lane < cnt ? a.col_idx[base + lane] : -1;
    // Q and the list are consumed here, before any copy is in flight, so the
    // compiler's own load waits never stall on a tile.
#pragma unroll
    for (int k = 0; k < D / 16; ++k) sa::keep(qr[k]);
    sa::keep(lst);
    if (!first_pass) ring_barrier();  // every wave is done with the rings
    first_pass = false;

    const int T = cnt * C::SUBS;       // 64-key tiles of this pass
    const int NI = (T + np - 1) / np;  // pipeline steps of each group

    // Key block of this group's tile at step m, or -1 when the tile is past
    // the end of the pass or its id is outside [0, limit) (such tiles are
    // loaded from a safe block and fully masked).
    auto tile_kb = [&](int m) -> int32_t {
      const int t = m * np + gs;
      const int32_t kb = sa::readlane(lst, min(t, T - 1) / C::SUBS);
      return (t < T && (uint32_t)kb < (uint32_t)limit) ? kb : -1;
    };
    auto tile_sub = [&](int m) -> int { return C::SUBS == 1 ? 0 : min(m * np + gs, T - 1) % C::SUBS; };
    auto dma_k = [&](int m, int32_t kb, int slot) {
      dma_tile(K, kbs, ks2, offK, offK1, offK4, k_contig, kring, slot, kb < 0 ? it.i : kb, tile_sub(m));
    };
    auto dma_v = [&](int m, int32_t kb, int slot) {
      dma_tile(V, vbs, vs2, offV, offV1, offV4, v_contig, vring, slot, kb < 0 ? it.i : kb, tile_sub(m));
    };
    // K operand of S^T = K Q^T for k-step k: 32 keys (kt) x 16 dims.
    auto k_operand = [&](const uint8_t* ks, int k, int kt) -> sa::u32x4 {
      const int key = 32 * kt + lq;
      return *(const sa::u32x4*)(ks + key * C::ROWB + sa::lds_slot<D>(2 * k + hl, key) * 16);
    };

    // S^T = K Q^T of the one slot, operand m = 2 k + kt read kKAhead MFMAs
    // before its use (sched barriers keep that order; the compiler counts the
    // reads when it places the waits).
    auto qk_hand = [&](sa::f32x16(&dst)[2]) {
      constexpr int NS = 2 * (D / 16);
      constexpr int R = kKAhead < NS ? kKAhead : NS;
      sa::u32x4 buf[NS];
      auto rd = [&](auto m) {
        constexpr int M = decltype(m)::value;
        buf[M] = *(const sa::u32x4*)(kop_p[M >> 1] + (M & 1) * 32 * C::ROWB);
      };
      sa::static_for<0, R>(rd);
      sa::static_for<0, NS>([&](auto m) {
        constexpr int M = decltype(m)::value;
        SA_SCHED_BARRIER();
        dst[M & 1] = M < 2 ? sa::mfma32_z(buf[M], qr[M >> 1]) : sa::mfma32(buf[M], qr[M >> 1], dst[M & 1]);
        if constexpr (M + R < NS) rd(std::integral_constant<int, M + R>{});
      });
      SA_SCHED_BARRIER();
    };
    auto qk = [&](const uint8_t* ks, sa::f32x16(&dst)[2]) {
#pragma unroll
      for (int k = 0; k < D / 16; ++k)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          dst[kt] = k == 0 ? sa::mfma32_z(k_operand(ks, k, kt), qr[k])
                           : sa::mfma32(k_operand(ks, k, kt), qr[k], dst[kt]);
    };

    // Key blocks of the tiles whose copies are in flight (q0 = step n).
    int32_t q0 = tile_kb(0), q1 = NI > 1 ? tile_kb(1) : -1, q2 = S > 2 && NI > 2 ? tile_kb(2) : -1;
    if constexpr (PIPE) {
      // prologue: K(0), then {K(j), V(j-1)} for j < S; S(0) = K(0) Q^T
      dma_k(0, q0, 0);
      if (1 < NI) dma_k(1, q1, 1);
      dma_v(0, q0, 0);
      if (S > 2) {
        if (2 < NI) dma_k(2, q2, 2 % S);
        if (1 < NI) dma_v(1, q1, 1);
      }
      int c = 0;
#pragma unroll
      for (int j = 1; j < S; ++j) c += (j < NI) + (j - 1 < NI);
      wait_vm_units<C::JN>(c);
      ring_barrier();
      qk(kring_p, sA);
    } else {
      // prologue: {K(j), V(j)} for j < S - 1
      dma_k(0, q0, 0);
      dma_v(0, q0, 0);
      if (S > 2 && 1 < NI) {
        dma_k(1, q1, 1);
        dma_v(1, q1, 1);
      }
    }

    // One pipeline step: softmax + O update of tile n (logits in `cur`), and,
    // when NEXT, the logits of tile n + 1 into `nxt`.
    auto step = [&](int n, sa::f32x16(&cur)[2], sa::f32x16(&nxt)[2], auto next_tag, auto par_tag) {
      constexpr bool NEXT = decltype(next_tag)::value;
      // ring slot of tile n (a compile-time constant when the caller passes
      // the parity of n and there are two slots)
      constexpr int PAR = decltype(par_tag)::value;
      const int pn = S == 2 && PAR >= 0 ? PAR : n % S;
      SA_SCHED_BARRIER();  // the previous step's MFMAs are issued before this wait
      int32_t qn = -1;  // key block of the newest tile put in flight
      // V^T operands of the one-slot kernels, j = u (D / 32) + dt: keys
      // 16 u .. 16 u + 15, d-columns 32 dt .. 32 dt + 31
      constexpr int NV = 4 * (D / 32);
      sa::u32x4 vbuf[NV];
      auto vread = [&](auto j) {
        constexpr int J = decltype(j)::value, U = J / (D / 32), DT = J % (D / 32);
        const sa::u32x2 lo = sa::lds_read_tr16(vop_p[DT] + U * 16 * C::ROWB);
        const sa::u32x2 hi = sa::lds_read_tr16(vop_p[DT] + U * 16 * C::ROWB + 8 * C::ROWB);
        vbuf[J] = sa::u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      if constexpr (PIPE) {
        // K(n+1) and V(n) must have landed (all waves): wait for the copies
        // issued up to step n+1-S; the barrier then also frees K(n), V(n-1).
        if (S == 3)
          wait_vm_units<C::JN>((n + 2 < NI) + (n + 1 < NI));
        else
          wait_vmcnt<0>();
        ring_barrier();
        if (n + S < NI) {
          qn = tile_kb(n + S);
          dma_k(n + S, qn, pn);
        }
        if (n + S - 1 < NI) dma_v(n + S - 1, S > 2 ? q2 : q1, (pn + S - 1) % S);
      } else if constexpr (S == 1) {
        // K(n) and V(n) must have landed (copied at the end of step n-1)
        wait_vmcnt<0>();
        ring_barrier();
        qk_hand(cur);
        sa::static_for<0, kVAhead>(vread);  // in flight during the softmax
      } else {
        // K(n) and V(n) must have landed; the barrier also frees tile n-1
        if (S == 3)
          wait_vm_units<C::JN>(2 * (n + 1 < NI));
        else
          wait_vmcnt<0>();
        ring_barrier();
        if (n + S - 1 < NI) {
          qn = tile_kb(n + S - 1);
          dma_k(n + S - 1, qn, (pn + S - 1) % S);
          dma_v(n + S - 1, qn, (pn + S - 1) % S);
        }
        qk(kring_p + pn * C::SLOTB, cur);
      }

      const uint8_t* ks = kring_p + ((pn + 1) % S) * C::SLOTB;  // K(n+1) (PIPE only)
      const uint8_t* vs = vring_p + pn * C::SLOTB;
      sa::u32x4 kop[C::KPA][2];
      if constexpr (NEXT) {
#pragma unroll
        for (int k = 0; k < C::KPRE; ++k)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) kop[k][kt] = k_operand(ks, k, kt);
      }

      // masking of tile n: the diagonal block (keys after the query) and
      // skipped tiles (everything) get -inf logits
      const int32_t kb = q0;
      const int sub_local = 64 * tile_sub(n);
      if (kb < 0 || (a.causal && kb == it.i && sub_local + 63 > wq * 32)) {
        // element (kt, e) holds key 32 kt + 8 (e / 4) + 4 hl + e % 4 of the tile
        const int lim = (kb < 0 ? -1 : q_local - sub_local) - 4 * hl;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            cur[kt][e] = 32 * kt + 8 * (e >> 2) + (e & 3) > lim ? -INFINITY : cur[kt][e];
      }
      // advance the key-block queue
      if constexpr (PIPE) {
        q0 = q1;
        if (S > 2) {
          q1 = q2;
          q2 = qn;
        } else {
          q1 = qn;
        }
      } else {
        if (S > 2) {
          q0 = q1;
          q1 = qn;
        } else if (S == 2) {
          q0 = qn;
        }  // one slot: q0 moves on at the end of the step
      }

      // tile max over both half-rows, in log2 units (max3 chains)
      float r[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const sa::f32x16& x = cur[c >> 1];
        const int o = 8 * (c & 1);
        float v = fmaxf(fmaxf(x[o], x[o + 1]), x[o + 2]);
        v = fmaxf(fmaxf(v, x[o + 3]), x[o + 4]);
        r[c] = fmaxf(fmaxf(v, x[o + 5]), x[o + 6]);
      }
      float rm = fmaxf(fmaxf(r[0], r[1]), r[2]);
      rm = fmaxf(fmaxf(rm, r[3]), cur[0][7]);
      rm = fmaxf(fmaxf(rm, cur[0][15]), cur[1][7]);
      rm = sa::max_xor32(fmaxf(rm, cur[1][15]));
      const float m_tile = rm * c2;
      const bool need = m_tile > m_used + kTau;
      if (__ballot(need)) {  // some query's max grew: move its reference
        const float m_new = need ? m_tile : m_used;
        const float alpha = sa::fast_exp2(m_used - m_new);
#pragma unroll
        for (int w = 0; w < 4; ++w) ls[w] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
        m_used = m_new;
      }

      // S(n+1) MFMAs (issued first, they run while the VALU works on P(n))
      if constexpr (NEXT) {
#pragma unroll
        for (int k = 0; k < D / 16; ++k)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const sa::u32x4 av = k < C::KPRE ? kop[k < C::KPRE ? k : 0][kt] : k_operand(ks, k, kt);
            nxt[kt] = k == 0 ? sa::mfma32_z(av, qr[k]) : sa::mfma32(av, qr[k], nxt[kt]);
          }
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
            pb[2 * kt + h2][w] = sa::pack_bf16x2(sa::fast_exp2(__builtin_fmaf(cur[kt][e], c2, -m_used)),
                                                 sa::fast_exp2(__builtin_fmaf(cur[kt][e + 1], c2, -m_used)));
          }
      if constexpr (kHand) {
        // O^T += V^T P^T, operands read kVRing MFMAs ahead; then the row sums
        // over the rounded P actually fed to the MFMA, on the VALU while the
        // last MFMAs run
        sa::static_for<kVAhead, kVRing>(vread);
        sa::static_for<0, NV>([&](auto j) {
          constexpr int J = decltype(j)::value;
          SA_SCHED_BARRIER();
          oacc[J % (D / 32)] = sa::mfma32(vbuf[J], pb[J / (D / 32)], oacc[J % (D / 32)]);
          if constexpr (J + kVRing < NV) vread(std::integral_constant<int, J + kVRing>{});
        });
        SA_SCHED_BARRIER();
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int w = 0; w < 4; ++w) ls[0] = sa::dot2_bf16(pb[u][w], 0x3f803f80u, ls[0]);
        if (n + 1 < NI) {
          // every wave has read tile n (its LDS reads returned): refill the slots
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          ring_barrier();
          q0 = tile_kb(n + 1);
          dma_k(n + 1, q0, 0);
          dma_v(n + 1, q0, 0);
        }
        return;
      }
      // row sums over the rounded P actually fed to the MFMA
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) ls[w] = sa::dot2_bf16(pb[u][w], 0x3f803f80u, ls[w]);
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
          const sa::u32x2 l2 = sa::lds_read_tr16(vs + keyA * C::ROWB + sa::lds_slot_tr<D>(cs, keyA) * 16 + half * 8);
          const sa::u32x2 h2 = sa::lds_read_tr16(vs + keyB * C::ROWB + sa::lds_slot_tr<D>(cs, keyB) * 16 + half * 8);
          const sa::u32x4 av = {l2[0], l2[1], h2[0], h2[1]};
          oacc[dt] = sa::mfma32(av, pb[u], oacc[dt]);
        }
      }
      // issue pattern: V operand reads first, then each S(n+1) MFMA followed by
      // a slice of the softmax VALU work, then the O MFMAs
      SA_SCHED_GROUP(0x100, 2 * (D / 32) * 4 + (NEXT ? 2 * (D / 16 - C::KPRE) : 0));
      if constexpr (NEXT) {
#pragma unroll
        for (int x = 0; x < 2 * (D / 16); ++x) {
          SA_SCHED_GROUP(0x008, 1);
          SA_SCHED_GROUP(0x002, kVGroup);
        }
      }
      SA_SCHED_GROUP(0x002, 128);
      SA_SCHED_GROUP(0x008, 4 * (D / 32));
      if constexpr (!PIPE && S == 1) {
        if (n + 1 < NI) {
          // every wave has read tile n (its LDS reads returned): refill the slots
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          ring_barrier();
          q0 = tile_kb(n + 1);
          dma_k(n + 1, q0, 0);
          dma_v(n + 1, q0, 0);
        }
      }
    };

    using yes = std::true_type;
    using no = std::false_type;
    using even = std::integral_constant<int, 0>;
    using odd = std::integral_constant<int, 1>;
    int n = 0;
    if constexpr (PIPE) {
      for (; n + 2 < NI; n += 2) {
        step(n, sA, sB, yes{}, even{});
        step(n + 1, sB, sA, yes{}, odd{});
      }
      if (n + 1 < NI) {
        step(n, sA, sB, yes{}, even{});
        step(n + 1, sB, sA, no{}, odd{});
      } else {
        step(n, sA, sB, no{}, even{});
      }
    } else {
      for (; n < NI; ++n) step(n, sA, sB, no{}, std::integral_constant<int, -1>{});
    }
  }
  float l_run = (ls[0] + ls[1]) + (ls[2] + ls[3]);

  // merge the groups' partial states into group 0
  l_run = sa::sum_xor32(l_run);

  // Part of a split row: publish this part's state (O^T partial, m, l; per
  // wave, element-major so each store covers 64 consecutive floats), then count
  // the arrival.  The last of the W parts to arrive merges the W states, read
  // back in part order so the result does not depend on the arrival order,
  // finishes the row and sets the counter back to 0 for the next launch.  The
  // states go through device-scope stores and loads (written through to, and
  // read from, the device coherence point) rather than fences, which would
  // write back and invalidate the whole L2 that the other workgroups of the XCD
  // are reading K and V from.
  if (NP == 1 && part >= 0) {
    constexpr int PER = D / 2 + 2;
    constexpr int64_t SLOTF = (int64_t)C::QW * PER * 64;  // floats per partial state
    const int W = a.split_ways;
    const int64_t row = (int64_t)unit_bh * a.split_rows + unit_pos;
    float* const states = a.split_part + row * W * SLOTF + (int64_t)wq * PER * 64 + lane;
    float* mine = states + part * SLOTF;
    auto publish = [](float* p, float x) { __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    auto fetch = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) publish(mine + (16 * dt + e) * 64, oacc[dt][e]);
    publish(mine + (D / 2) * 64, m_used);
    publish(mine + (D / 2 + 1) * 64, l_run);
    wait_vmcnt<0>();  // this wave's stores have reached the coherence point
    __syncthreads();  // ... and the other waves'; every wave is past its last tile
    int* arrival = (int*)smem;
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(a.split_cnt + row, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == W - 1) __hip_atomic_store(a.split_cnt + row, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      arrival[0] = old;
    }
    __syncthreads();
    if (arrival[0] != W - 1) return;
    m_used = fetch(states + (D / 2) * 64);
    l_run = fetch(states + (D / 2 + 1) * 64);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][e] = fetch(states + (16 * dt + e) * 64);
    for (int p = 1; p < W; ++p) {
      const float* st = states + p * SLOTF;
      const float mo = fetch(st + (D / 2) * 64), lo = fetch(st + (D / 2 + 1) * 64);
      const float mm = fmaxf(m_used, mo);
      const float a0 = sa::fast_exp2(m_used - mm), a1 = sa::fast_exp2(mo - mm);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = oacc[dt][e] * a0 + fetch(st + (16 * dt + e) * 64) * a1;
      l_run = l_run * a0 + lo * a1;
      m_used = mm;
    }
  }
  if constexpr (NP > 1) {
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the rings; reuse them
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
      const float a0 = sa::fast_exp2(m_used - mm), a1 = sa::fast_exp2(mo - mm);
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

// (groups per workgroup NP, ring slots S, software-pipelined S(n+1)) of each
// compiled tile shape.  One slot, not pipelined, for whole rows: 4 % (long rows)
// to 12 % faster than a two-slot ring on the compression-guided, gzip-guided
// and long-context masks, from the higher occupancy
#define SA_CFG_WHOLE 1, 1, false
// ... and with each row split over two wave groups (row_split = 2): a two-slot
// ring, software-pipelined at d = 64 (at d = 128 the pipelined form needs more
// than 256 registers)
#define SA_CFG_SPLIT64 2, 2, true
#define SA_CFG_SPLIT128 2, 2, false

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
    const int64_t grid = (int64_t)a.B * a.H * (a.nb + (int64_t)a.split_rows * (a.split_ways - 1)); \
    hipLaunchKernelGGL((bsa_fwd_bf16_kernel<D, BLK, CFG>), dim3((unsigned)grid), dim3(Cf::NT), \
                       Cf::LDSB, stream, a);                                                 \
    return sa_host::check_launch(NAME);                                                      \
  } while (0)

// Split-row workspace: a counter area of fixed size (SA_SPLIT_COUNTERS int32,
// whatever the split shape, so that launches of any shape that share a
// workspace find their counters at zero), then the partial states of every
// part of every split row.
struct SplitLayout {
  int64_t part, total;
};
inline SplitLayout split_layout(int64_t B, int64_t H, int64_t d, int64_t block, int64_t split_rows,
                                int64_t split_ways) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  SplitLayout l;
  l.part = (int64_t)SA_SPLIT_COUNTERS * 4;
  l.total = split_rows > 0 ? l.part + up(B * H * split_rows * split_ways * (block / 32) * 64 * (d / 2 + 2) * 4)
                           : 0;
  return l;
}

// Checks every argument of sparse_attn_fwd and fills the kernel arguments;
// nothing is launched.  The workspace pointer is only checked and stored.
sa_status fwd_setup(int32_t dtype, const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                    int32_t H, int32_t H_kv, int32_t N, int32_t d, int32_t block, const int64_t* strides,
                    const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity, const int32_t* sched,
                    int32_t num_groups, int64_t mask_batch_stride, int64_t mask_head_stride, int32_t causal,
                    float scale, int32_t row_split, int32_t split_rows, int32_t split_ways, void* workspace,
                    int64_t workspace_bytes, BsaArgs& a) {
  if (!q || !k || !v || !o || !lse || !row_ptr || !col_idx) return SA_ERR_NULL;
  if (row_split != 1 && row_split != 2) return SA_ERR_INVALID;
  if (split_rows < 0) return SA_ERR_INVALID;
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
  if (split_rows > nb) return SA_ERR_INVALID;
  // split rows apply to the bf16 whole-row kernels; the fp32 path ignores them
  const int32_t splits = dtype == SA_BF16 ? split_rows : 0;
  if (splits > 0 && row_split != 1) return SA_ERR_INVALID;
  if (splits > 0 && (split_ways < 2 || split_ways > SA_MAX_SPLIT_WAYS)) return SA_ERR_INVALID;
  const int32_t ways = splits > 0 ? split_ways : 1;
  if ((int64_t)B * H * splits > SA_SPLIT_COUNTERS) return SA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * (nb + (int64_t)splits * (ways - 1)) > 0x7fffffffll) return SA_ERR_UNSUPPORTED;
  const SplitLayout sl = split_layout(B, H, d, block, splits, ways);
  if (splits > 0) {
    if (!workspace) return SA_ERR_NULL;
    if (!sa_host::aligned16(workspace)) return SA_ERR_INVALID;
    if (workspace_bytes < sl.total) return SA_ERR_CAPACITY;
  }
  if (!sa_host::aligned16(q) || !sa_host::aligned16(k) || !sa_host::aligned16(v) ||
      !sa_host::aligned16(o))
    return SA_ERR_INVALID;
  sa_host::Strides st[4];
  const sa_status ss = sa_host::resolve_strides(strides, B, H, H_kv, N, d, dtype == SA_BF16 ? 8 : 4, st);
  if (ss != SA_OK) return ss;
  // the bf16 kernel keeps the byte offsets of the rows of a 64-key tile in 32 bits
  if (dtype == SA_BF16 && (st[1].s >= (int64_t)1 << 24 || st[2].s >= (int64_t)1 << 24))
    return SA_ERR_UNSUPPORTED;

  a = BsaArgs{};
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
  a.scale_log2 = scale != 0.f ? fabsf(scale) * sa::kLog2e : 1e-30f;
  a.qsign = scale < 0.f ? 0x80008000u : 0u;
  a.split_rows = splits;
  a.split_ways = ways;
  a.split_cnt = splits > 0 ? (int32_t*)workspace : nullptr;
  a.split_part = splits > 0 ? (float*)((uint8_t*)workspace + sl.part) : nullptr;
  return SA_OK;
}

// Launch of the kernel that serves (dtype, d, block, row_split).
sa_status fwd_launch(const BsaArgs& a, int32_t dtype, int32_t d, int32_t block, int32_t row_split,
                     hipStream_t stream) {
  if (dtype == SA_BF16 && row_split == 2) {
    if (d == 64 && block == 64) SA_LAUNCH_BF16(64, 64, SA_CFG_SPLIT64, "bsa_fwd_bf16<64,64,split>");
    if (d == 64 && block == 128) SA_LAUNCH_BF16(64, 128, SA_CFG_SPLIT64, "bsa_fwd_bf16<64,128,split>");
    if (d == 128 && block == 64) SA_LAUNCH_BF16(128, 64, SA_CFG_SPLIT128, "bsa_fwd_bf16<128,64,split>");
    SA_LAUNCH_BF16(128, 128, SA_CFG_SPLIT128, "bsa_fwd_bf16<128,128,split>");
  }
  if (dtype == SA_BF16) {
    if (d == 64 && block == 64) SA_LAUNCH_BF16(64, 64, SA_CFG_WHOLE, "bsa_fwd_bf16<64,64>");
    if (d == 64 && block == 128) SA_LAUNCH_BF16(64, 128, SA_CFG_WHOLE, "bsa_fwd_bf16<64,128>");
    if (d == 128 && block == 64) SA_LAUNCH_BF16(128, 64, SA_CFG_WHOLE, "bsa_fwd_bf16<128,64>");
    SA_LAUNCH_BF16(128, 128, SA_CFG_WHOLE, "bsa_fwd_bf16<128,128>");
  }
  if (d == 64 && block == 64) return launch(bsa_fwd_f32_kernel<64, 64>, a, 64, 0, stream, "bsa_fwd_f32<64,64>");
  if (d == 64 && block == 128) return launch(bsa_fwd_f32_kernel<64, 128>, a, 128, 0, stream, "bsa_fwd_f32<64,128>");
  if (d == 128 && block == 64) return launch(bsa_fwd_f32_kernel<128, 64>, a, 64, 0, stream, "bsa_fwd_f32<128,64>");
  return launch(bsa_fwd_f32_kernel<128, 128>, a, 128, 0, stream, "bsa_fwd_f32<128,128>");
}

// Scratch of sparse_attn_fwd_noalloc: the split-row workspace of callers that
// cannot allocate.  Every device holds its own copy until the process ends;
// host code reaches it only through the address hipGetSymbolAddress returns
// for the current device (the array's name is a host-side stand-in).
static __device__ __align__(256) uint8_t scratch[SA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
sa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sa_host::record_hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return sa_host::record_hip_error(e, "hipGetSymbolAddress(scratch)");
    if (!p) return SA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

// Sets n int32 to zero (a kernel rather than a memset, so that the call can
// sit in a captured graph).
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* p, int32_t n) {
  const int32_t x = blockIdx.x * 256 + threadIdx.x;
  if (x < n) p[x] = 0;
}

}  // namespace

extern "C" int64_t sparse_attn_fwd_workspace_bytes(int32_t B, int32_t H, int32_t d, int32_t block,
                                                   int32_t split_rows, int32_t split_ways) {
  if (B < 1 || H < 1 || split_rows < 0) return SA_ERR_INVALID;
  if (split_rows > 0 && (split_ways < 2 || split_ways > SA_MAX_SPLIT_WAYS)) return SA_ERR_INVALID;
  if ((d != 64 && d != 128) || (block != 64 && block != 128)) return SA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * split_rows > SA_SPLIT_COUNTERS) return SA_ERR_UNSUPPORTED;
  return split_layout(B, H, d, block, split_rows, split_ways).total;
}

extern "C" sa_status sparse_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                                     void* o, float* lse, int32_t B, int32_t H, int32_t H_kv,
                                     int32_t N, int32_t d, int32_t block, const int64_t* strides,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t col_capacity, const int32_t* sched, int32_t num_groups,
                                     int64_t mask_batch_stride, int64_t mask_head_stride,
                                     int32_t causal, float scale, int32_t row_split, int32_t split_rows,
                                     int32_t split_ways, void* workspace, int64_t workspace_bytes,
                                     hipStream_t stream) {
  BsaArgs a;
  const sa_status st = fwd_setup(dtype, q, k, v, o, lse, B, H, H_kv, N, d, block, strides, row_ptr, col_idx,
                                 col_capacity, sched, num_groups, mask_batch_stride, mask_head_stride, causal,
                                 scale, row_split, split_rows, split_ways, workspace, workspace_bytes, a);
  if (st != SA_OK) return st;
  return fwd_launch(a, dtype, d, block, row_split, stream);
}

extern "C" sa_status sparse_attn_fwd_noalloc(int32_t dtype, const void* q, const void* k, const void* v,
                                             void* o, float* lse, int32_t B, int32_t H, int32_t H_kv,
                                             int32_t N, int32_t d, int32_t block, const int64_t* strides,
                                             const int32_t* row_ptr, const int32_t* col_idx,
                                             int64_t col_capacity, const int32_t* sched, int32_t num_groups,
                                             int64_t mask_batch_stride, int64_t mask_head_stride,
                                             int32_t causal, float scale, int32_t row_split,
                                             int32_t split_rows, int32_t split_ways, hipStream_t stream) {
  const bool uses = dtype == SA_BF16 && split_rows > 0;
  if (uses) {
    const int64_t need = sparse_attn_fwd_workspace_bytes(B, H, d, block, split_rows, split_ways);
    if (need > SA_NOALLOC_SCRATCH_BYTES) return SA_ERR_CAPACITY;
  }
  // every argument is checked before the scratch is looked up or anything is
  // launched (a placeholder address stands in for the scratch while checking)
  BsaArgs a;
  sa_status st = fwd_setup(dtype, q, k, v, o, lse, B, H, H_kv, N, d, block, strides, row_ptr, col_idx,
                           col_capacity, sched, num_groups, mask_batch_stride, mask_head_stride, causal, scale,
                           row_split, split_rows, split_ways, uses ? (void*)(uintptr_t)256 : nullptr,
                           SA_NOALLOC_SCRATCH_BYTES, a);
  if (st != SA_OK) return st;
  if (uses) {
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != SA_OK) return st;
    a.split_cnt = (int32_t*)ws;
    a.split_part = (float*)((uint8_t*)ws + split_layout(B, H, d, block, a.split_rows, a.split_ways).part);
    // the counters this launch uses start at zero whatever an earlier call left
    const int32_t n = B * H * a.split_rows;
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.split_cnt, n);
    st = sa_host::check_launch("zero_i32_kernel");
    if (st != SA_OK) return st;
  }
  return fwd_launch(a, dtype, d, block, row_split, stream);
}
