// Device construction of the block-mask CSR: count -> prefix sum -> fill.
// Up to kDirectRows rows the prefix sum is folded into the fill: the counts go
// to scratch entries of col_idx past the largest possible CSR, and every fill
// workgroup sums the counts of the rows before its own (two launches instead
// of three).
//
// Row (g, i) of the mask is the union, in block units, of the identity, the
// local window, the global blocks, the random draws and the literal blocks
// ("Parameter-free Adaptive Sparse Attention via Compression-Based Content
// Selection", Sec. 3.2 Eq. 3; "BigBird", Sec. 2 graphs G_W, G_G, G_R),
// intersected with j <= i when causal.  One wave owns one row: lane l decides
// columns j = l, l + 64, ... and ballots give the count and the write
// positions, so the columns come out ascending without a sort.
#include <math.h>

#include "sa_device.h"
#include "sa_host.h"

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kScanThreads = 1024;
constexpr int64_t kDirectRows = 8192;

struct MaskArgs {
  int32_t nb, G, causal, wb, wa, clamp;
  int32_t num_global, num_random, lit_mode;
  int32_t excl;  // SA_PART_* bits left out of every group's union
  int32_t period;  // P > 0: per-group exclusions period_excl[g % P], flags row g / P
  int32_t period_excl[SA_MAX_PERIOD];
  int32_t globals[SA_MAX_GLOBAL];
  const int32_t* random_blocks;
  const uint8_t* lit_flags;
  uint64_t lit_thr;  // 0 .. 2^32
  uint64_t seed;
  int32_t* row_ptr;
  int32_t* col_idx;
  int64_t col_capacity;
  int32_t* sched;
  int32_t* counts;  // [G * nb] row lengths (direct mode), else nullptr
};

// Everything a wave needs to decide membership for one row.
struct RowCtx {
  int32_t g, i;
  int32_t fg;    // literal-flag group (g, or g / P)
  int32_t excl;  // components left out of this group's union
  bool valid;
  bool row_global;
  bool lit_i;
  uint64_t lit_key;  // key_prefix(seed, 1, flag group) of the literal draws
  int32_t ndraw;     // accepted random blocks, stored in LDS
};

__device__ __forceinline__ bool literal_of(const MaskArgs& a, const RowCtx& c, int32_t j) {
  if (a.lit_flags) return a.lit_flags[(int64_t)c.fg * a.nb + j] != 0;
  return sa::literal_draw(c.lit_key, (uint64_t)j, a.lit_thr);
}

__device__ __forceinline__ bool is_global(const MaskArgs& a, int32_t j) {
  bool hit = false;
  for (int n = 0; n < a.num_global; ++n) hit |= (a.globals[n] == j);
  return hit;
}

// Set up the row of this wave.  Lane 0 performs the random draws into `draws`.
// Must be called by every thread of the block (contains a barrier).
__device__ RowCtx setup_row(const MaskArgs& a, int64_t r, int32_t* draws, int lane) {
  RowCtx c;
  const int64_t R = (int64_t)a.G * a.nb;
  c.valid = r < R;
  c.g = c.valid ? (int32_t)(r / a.nb) : 0;
  c.i = c.valid ? (int32_t)(r - (int64_t)c.g * a.nb) : 0;
  c.fg = a.period > 0 ? c.g / a.period : c.g;
  c.excl = a.excl | (a.period > 0 ? a.period_excl[c.g % a.period] : 0);
  c.row_global = is_global(a, c.i);
  c.lit_key = sa::key_prefix(a.seed, sa::kTagLiteral, (uint64_t)c.fg);
  c.lit_i = (a.lit_mode != SA_LIT_NONE) && c.valid && literal_of(a, c, c.i);
  c.ndraw = 0;
  if (lane == 0 && c.valid && a.num_random > 0) {
    const int32_t n = a.causal ? c.i : a.nb;
    const int32_t want = min(a.num_random, n);
    int32_t cnt = 0;
    if (a.random_blocks) {
      const int32_t* src = a.random_blocks + r * a.num_random;
      for (int k = 0; k < a.num_random; ++k) {
        const int32_t x = src[k];
        if (x < 0 || x >= n) continue;
        bool seen = false;
        for (int m = 0; m < cnt; ++m) seen |= (draws[m] == x);
        if (!seen) draws[cnt++] = x;
      }
    } else if (want > 0) {
      cnt = sa::draw_distinct(a.seed, (uint64_t)c.g, (uint64_t)c.i, n, a.num_random, draws);
    }
    draws[SA_MAX_RANDOM] = cnt;
  }
  __syncthreads();
  if (c.valid && a.num_random > 0) c.ndraw = draws[SA_MAX_RANDOM];
  return c;
}

__device__ __forceinline__ bool member(const MaskArgs& a, const RowCtx& c, const int32_t* draws,
                                       int32_t j) {
  const int32_t i = c.i;
  if (a.causal && j > i) return false;
  if (j == i) return true;
  // local window
  if (!(c.excl & SA_PART_WINDOW)) {
    if (a.causal) {
      if (j >= i - a.wb) return true;
    } else if (a.clamp) {
      const int32_t width = a.wb + a.wa + 1;
      if (width >= a.nb) return true;
      const int32_t start = min(max(i - a.wb, 0), a.nb - width);
      if (j >= start && j < start + width) return true;
    } else if (j >= i - a.wb && j <= i + a.wa) {
      return true;
    }
  }
  // global rows / columns
  if (!(c.excl & SA_PART_GLOBAL) && (c.row_global || is_global(a, j))) return true;
  // random draws
  if (!(c.excl & SA_PART_RANDOM))
    for (int m = 0; m < c.ndraw; ++m)
      if (draws[m] == j) return true;
  // literal blocks outside the window band
  if (!(c.excl & SA_PART_LITERAL) && a.lit_mode != SA_LIT_NONE && (j < i - a.wb || j > i + a.wa)) {
    if (a.lit_mode == SA_LIT_PAIR && !c.lit_i) return false;
    return literal_of(a, c, j);
  }
  return false;
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void mask_count_kernel(MaskArgs a) {
  __shared__ int32_t draws[kWavesPerBlock][SA_MAX_RANDOM + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const RowCtx c = setup_row(a, r, draws[wave], lane);
  if (!c.valid) return;
  int32_t count = 0;
  for (int32_t j0 = 0; j0 < a.nb; j0 += 64) {
    const int32_t j = j0 + lane;
    const bool m = j < a.nb && member(a, c, draws[wave], j);
    count += __popcll(__ballot(m));
  }
  if (lane == 0) {
    if (a.counts) {
      a.counts[r] = count;
    } else {
      a.row_ptr[r + 1] = count;
      if (r == 0) a.row_ptr[0] = 0;
    }
  }
}

// In-place inclusive prefix sum of row_ptr[1..R] (one block).
__global__ __launch_bounds__(kScanThreads) void mask_scan_kernel(MaskArgs a) {
  __shared__ int64_t part[kScanThreads];
  const int64_t R = (int64_t)a.G * a.nb;
  const int64_t chunk = (R + kScanThreads - 1) / kScanThreads;
  const int t = threadIdx.x;
  const int64_t beg = min(R, t * chunk), end = min(R, beg + chunk);
  int64_t s = 0;
  for (int64_t x = beg; x < end; ++x) s += a.row_ptr[x + 1];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {  // Hillis-Steele inclusive scan
    const int64_t add = (t >= off) ? part[t - off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int64_t run = part[t] - s;  // exclusive prefix of this chunk
  for (int64_t x = beg; x < end; ++x) {
    run += a.row_ptr[x + 1];
    a.row_ptr[x + 1] = (int32_t)run;
  }
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void mask_fill_kernel(MaskArgs a) {
  __shared__ int32_t draws[kWavesPerBlock][SA_MAX_RANDOM + 1];
  __shared__ int64_t wsum[kWavesPerBlock];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * kWavesPerBlock, r = r0 + wave;
  const int64_t R = (int64_t)a.G * a.nb;
  int64_t start = 0;
  if (a.counts) {
    // entries before this block's first row: the sum of the earlier counts
    int64_t s = 0;
    for (int64_t x = threadIdx.x; x < r0; x += 64 * kWavesPerBlock) s += a.counts[x];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) wsum[wave] = s;
    __syncthreads();
    for (int w = 0; w < kWavesPerBlock; ++w) start += wsum[w];
    for (int w = 0; w < wave; ++w)
      if (r0 + w < R) start += a.counts[r0 + w];
  }
  const RowCtx c = setup_row(a, r, draws[wave], lane);
  if (!c.valid) return;
  if (a.counts) {
    if (lane == 0) {
      a.row_ptr[r + 1] = (int32_t)(start + a.counts[r]);
      if (r == 0) a.row_ptr[0] = 0;
    }
  } else {
    start = a.row_ptr[r];
  }
  int32_t run = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int32_t j0 = 0; j0 < a.nb; j0 += 64) {
    const int32_t j = j0 + lane;
    const bool m = j < a.nb && member(a, c, draws[wave], j);
    const uint64_t bits = __ballot(m);
    if (m) {
      const int64_t pos = (int64_t)start + run + __popcll(bits & below);
      if (pos < a.col_capacity) a.col_idx[pos] = j;
    }
    run += __popcll(bits);
  }
  if (a.sched) {
    // rank of this row in the group's longest-first order (ties: lower id first)
    const int32_t* rp = a.row_ptr + (int64_t)c.g * a.nb;
    const int32_t* cn = a.counts ? a.counts + (int64_t)c.g * a.nb : nullptr;
    auto len = [&](int32_t x) { return cn ? cn[x] : rp[x + 1] - rp[x]; };
    const int32_t mine = len(c.i);
    int32_t rank = 0;
    for (int32_t x = lane; x < a.nb; x += 64) {
      const int32_t other = len(x);
      rank += (other > mine) || (other == mine && x < c.i);
    }
    for (int off = 32; off > 0; off >>= 1) rank += __shfl_xor(rank, off);
    if (lane == 0) a.sched[(int64_t)c.g * a.nb + rank] = c.i;
  }
}

// floor(p * 2^32) in double, clamped to [0, 2^32] (0 for p <= 0 or NaN).
uint64_t literal_threshold(double p) {
  const double t = floor(p * 4294967296.0);
  return (p > 0.0) ? (uint64_t)fmin(t, 4294967296.0) : 0ull;
}

// Largest possible number of CSR entries.
int64_t entry_bound(const sa_mask_desc* d) {
  const int64_t G = d->num_groups, nb = d->num_blocks;
  return d->causal ? G * nb * (nb + 1) / 2 : G * nb * nb;
}

sa_status check_desc(const sa_mask_desc* d) {
  if (d == nullptr) return SA_ERR_NULL;
  if (d->num_blocks < 1 || d->num_blocks > SA_MAX_BLOCKS) return SA_ERR_INVALID;
  if (d->num_groups < 1) return SA_ERR_INVALID;
  if ((int64_t)d->num_groups * d->num_blocks > (1ll << 24)) return SA_ERR_UNSUPPORTED;
  if (d->causal != 0 && d->causal != 1) return SA_ERR_INVALID;
  if (d->win_before < 0 || d->win_after < 0) return SA_ERR_INVALID;
  if (d->causal && d->win_after != 0) return SA_ERR_INVALID;
  if (d->win_clamp != 0 && d->win_clamp != 1) return SA_ERR_INVALID;
  if (d->num_global < 0 || d->num_global > SA_MAX_GLOBAL) return SA_ERR_INVALID;
  if (d->num_global > 0 && d->global_blocks == nullptr) return SA_ERR_NULL;
  for (int n = 0; n < d->num_global; ++n) {
    const int32_t x = d->global_blocks[n];
    if (x < 0 || x >= d->num_blocks) return SA_ERR_INVALID;
    if (n > 0 && x <= d->global_blocks[n - 1]) return SA_ERR_INVALID;
  }
  if (d->num_random < 0 || d->num_random > SA_MAX_RANDOM) return SA_ERR_INVALID;
  if (d->literal_mode < SA_LIT_NONE || d->literal_mode > SA_LIT_ANYQ) return SA_ERR_INVALID;
  if (d->exclude_parts < 0 || d->exclude_parts > 15) return SA_ERR_INVALID;
  if (d->group_period < 0 || d->group_period > SA_MAX_PERIOD) return SA_ERR_INVALID;
  for (int n = 0; n < d->group_period; ++n)
    if (d->period_exclude[n] < 0 || d->period_exclude[n] > 15) return SA_ERR_INVALID;
  if (d->literal_mode != SA_LIT_NONE && d->literal_flags == nullptr &&
      !(d->literal_p >= 0.0 && d->literal_p <= 1.0))
    return SA_ERR_INVALID;
  if (entry_bound(d) + (int64_t)d->num_groups * d->num_blocks > 0x7fffffffll) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

}  // namespace

extern "C" {

sa_status sparse_attn_check_mask_desc(const sa_mask_desc* desc) { return check_desc(desc); }

int64_t sparse_attn_mask_capacity(const sa_mask_desc* d) {
  const sa_status st = check_desc(d);
  if (st != SA_OK) return st;
  return entry_bound(d) + (int64_t)d->num_groups * d->num_blocks;  // + scratch for the row lengths
}

sa_status sparse_attn_build_mask(const sa_mask_desc* d, int32_t* row_ptr, int32_t* col_idx,
                                 int64_t col_capacity, int32_t* sched, hipStream_t stream) {
  const sa_status st = check_desc(d);
  if (st != SA_OK) return st;
  if (row_ptr == nullptr || col_idx == nullptr) return SA_ERR_NULL;
  if (col_capacity < sparse_attn_mask_capacity(d)) return SA_ERR_CAPACITY;
  if (d->num_random > 0 && d->random_blocks == nullptr) {
    // seeded draws: nothing to check
  }
  MaskArgs a = {};
  a.nb = d->num_blocks;
  a.G = d->num_groups;
  a.causal = d->causal;
  a.wb = d->win_before;
  a.wa = d->win_after;
  a.clamp = d->causal ? 0 : d->win_clamp;
  a.num_global = d->num_global;
  for (int n = 0; n < d->num_global; ++n) a.globals[n] = d->global_blocks[n];
  a.num_random = d->num_random;
  a.random_blocks = d->random_blocks;
  a.lit_mode = d->literal_mode;
  a.lit_flags = d->literal_flags;
  a.excl = d->exclude_parts;
  a.period = d->group_period;
  for (int n = 0; n < d->group_period; ++n) a.period_excl[n] = d->period_exclude[n];
  a.lit_thr = literal_threshold(d->literal_p);
  a.seed = d->seed;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_capacity = col_capacity;
  a.sched = sched;
  const int64_t R = (int64_t)a.G * a.nb;
  a.counts = R <= kDirectRows ? col_idx + entry_bound(d) : nullptr;
  const unsigned grid = (unsigned)((R + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(mask_count_kernel, dim3(grid), dim3(64 * kWavesPerBlock), 0, stream, a);
  sa_status e = sa_host::check_launch("mask_count_kernel");
  if (e != SA_OK) return e;
  if (!a.counts) {
    hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
    e = sa_host::check_launch("mask_scan_kernel");
    if (e != SA_OK) return e;
  }
  hipLaunchKernelGGL(mask_fill_kernel, dim3(grid), dim3(64 * kWavesPerBlock), 0, stream, a);
  return sa_host::check_launch("mask_fill_kernel");
}

uint64_t sa_rng_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c) {
  return sa::key_finish(sa::key_prefix(seed, tag, a), b, c);
}

int32_t sa_rng_literal(uint64_t seed, uint64_t group, uint64_t block, double p) {
  return sa::literal_draw(sa::key_prefix(seed, sa::kTagLiteral, group), block, literal_threshold(p)) ? 1 : 0;
}

int32_t sa_rng_random_blocks(uint64_t seed, uint64_t group, uint64_t row, int32_t n, int32_t r, int32_t* out) {
  if (out == nullptr) return SA_ERR_NULL;
  if (n < 0 || r < 0 || r > SA_MAX_RANDOM) return SA_ERR_INVALID;
  return sa::draw_distinct(seed, group, row, n, r, out);
}

}  // extern "C"
