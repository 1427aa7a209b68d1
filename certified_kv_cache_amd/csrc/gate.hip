// Meter-driven gate: pick blocks to repair and page their exact keys in.
//
// WitCert summary (implementation paragraph): a gate pages in exact blocks
// from a CPU backing store when the meter exceeds a threshold; paperswithlean
// Figure 2 caption: it repairs at block granularity from the exact store and
// zeroes the repaired witnesses; Figure 5 caption: risk-ranked where the
// witness is saturated (tau >= 1), certified where it is informative
// (tau < 1), incremental persistent repair.
//
// R = E (1 + E/2) <= tau is E <= E_tau = sqrt(1 + 2 tau) - 1.  Risks are
// turned into 40-bit fixed point so every decision is integer arithmetic
// and does not depend on summation order.
//
// Kernels: (1) per (sequence, KV head): fixed-point risks of all the group's
// query heads summed in the workgroup, the trigger test on the sums, then
// (rarely) the candidates sorted by risk and per-head scans for the shortest
// sufficient prefix; (2) per (sequence, KV head) and copy lane: the pool
// slots of the pair from the exclusive prefix of the counts in (sequence,
// head) order (deterministic, no atomics), the pool counters updated by one
// workgroup, then each selected block copied from pinned host memory
// (zero-copy reads) into the bf16 pool, its witness zeroed and the block
// marked.  Kernel (1) keeps the pool counter's value from before the call in
// the workspace, which is all kernel (2) reads of it, so the one write of the
// counter races with no read.
//
// Sorting any number of blocks: the candidates are cut into tiles of 4096
// that are sorted in LDS (bitonic) and written to the workspace, then merged
// pairwise in the workspace (merge path: every thread finds its share of the
// output by a binary search on the two runs) until one run is left.
//
// The tanh gate (the page-in comparison of the summary): the bound
// tanh(max_t c_t / 2) is <= tau for every head exactly when no unrepaired
// token has c_t > c* = 2 artanh(tau), so kernel (1) is replaced by one that
// takes every unrepaired block whose largest bound over the group's heads
// exceeds c*, ranked by that bound; (2) is shared.
#include <math.h>

#include <mutex>

#include "wc_common.h"

namespace wc {

constexpr int kFxBits = 40;
constexpr uint64_t kFxCap = uint64_t(1) << 47;
constexpr int kTile = 4096;          // blocks sorted per LDS tile
constexpr int kMaxPages = 65536;     // block index in the low 16 bits of a sort key
constexpr int kGateThreads = 256;

struct GateArgs {
  const float* logrisk;
  const float* lse;
  const float* meter;     // nullable: merged meter R of the gate's tier, [B][Hq]
  const int32_t* page_table;
  const int32_t* ctx_len;
  uint64_t* fx;           // [B][Hq][max_pages], optional copy for the caller
  int32_t* sel;           // [B][Hkv][max_pages]
  int32_t* count;         // [B][Hkv]
  int64_t* pool_old;      // the pool counter before this call
  uint64_t* keys;         // [B][Hkv][max_pages] sort keys
  uint64_t* keys2;        // [B][Hkv][max_pages] merge buffer
  int B, Hq, G, max_pages, layer;
  uint64_t T;
  float e_tau;            // E_tau rounded down to float (the quiet test)
  int64_t budget;
};

// rho_fx = ceil(rho 2^40) capped at 2^47, rho = e^(logrisk - lse).  rho
// 2^40 is an exact float (a power-of-two scaling below 2^47), so ceilf is
// exact and the 64-bit integer is assembled from two exact 32-bit parts.
__device__ __forceinline__ uint64_t risk_fx(float logrisk, float lse) {
  if (!(logrisk > -INFINITY)) return 0;                 // -inf (no risk) or NaN
  const float rho = __expf(logrisk - lse);
  if (!(rho < 128.0f)) return kFxCap;                   // >= 2^47 / 2^40, inf
  if (!(rho > 0.0f)) return 0;
  const float x = ceilf(rho * 1099511627776.0f);        // integer valued, < 2^47
  const float hi = floorf(x * 2.3283064365386963e-10f); // x / 2^32
  const float lo = x - hi * 4294967296.0f;
  const uint64_t u = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
  return u > kFxCap ? kFxCap : u;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Bitonic sort of keys[0 .. np2) (np2 a power of two) in LDS, descending;
// every thread of the workgroup calls it.
__device__ void sort_desc(uint64_t* keys, int np2, int t) {
  for (int kk = 2; kk <= np2; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = t; i < np2; i += kGateThreads) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const bool desc = (i & kk) == 0;
          const uint64_t x = keys[i], y = keys[ixj];
          if (desc ? (x < y) : (x > y)) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Elements of the descending run A among the first d outputs of the merge of
// A (length a) and B (length b), ties to A.
__device__ __forceinline__ int merge_split(const uint64_t* A, int a, const uint64_t* B, int b, int d) {
  int lo = d > b ? d - b : 0, hi = d < a ? d : a;
  while (lo < hi) {
    const int m = (lo + hi) >> 1;
    if (A[m] >= B[d - 1 - m]) lo = m + 1; else hi = m;
  }
  return lo;
}

// Sort the n keys that `key_of(j)` gives for j < n, descending, through the
// LDS tile `tile` and the two global buffers; returns the buffer holding the
// sorted keys.  Every thread of the workgroup calls it.
template <typename KeyOf>
__device__ uint64_t* sort_keys(int n, uint64_t* tile, uint64_t* buf0, uint64_t* buf1, int t, KeyOf key_of) {
  for (int base = 0; base < n; base += kTile) {
    const int len = min(kTile, n - base);
    int np2 = 1;
    while (np2 < len) np2 <<= 1;
    for (int i = t; i < np2; i += kGateThreads) tile[i] = i < len ? key_of(base + i) : 0;
    __syncthreads();
    sort_desc(tile, np2, t);
    for (int i = t; i < len; i += kGateThreads) buf0[base + i] = tile[i];
    __syncthreads();
  }
  uint64_t* src = buf0;
  uint64_t* dst = buf1;
  for (int w = kTile; w < n; w <<= 1) {
    __threadfence_block();
    __syncthreads();
    for (int lo = 0; lo < n; lo += 2 * w) {
      const int mid = min(lo + w, n), hi = min(lo + 2 * w, n);
      const int a = mid - lo, b = hi - mid, tot = a + b;
      const int per = (tot + kGateThreads - 1) / kGateThreads;
      const int d0 = min(tot, t * per), d1 = min(tot, d0 + per);
      if (d0 < d1) {
        const uint64_t* A = src + lo;
        const uint64_t* B = src + mid;
        int i = merge_split(A, a, B, b, d0), j = d0 - i;
        for (int d = d0; d < d1; ++d) {
          const bool takeA = i < a && (j >= b || A[i] >= B[j]);
          dst[lo + d] = takeA ? A[i++] : B[j++];
        }
      }
    }
    uint64_t* s = src;
    src = dst;
    dst = s;
  }
  __threadfence_block();
  __syncthreads();
  return src;
}

// Fixed-point risks, trigger test and (rarely) selection, one workgroup per
// (sequence, KV head).
//
// Quiet pairs: with the merged meter R_h given, E_h = 2 R_h / (sqrt(1 + 2 R_h) + 1)
// is the pair's head risk in float.  X_h / 2^40 is the same sum taken per block
// (every block rounded up by less than 2^-40) from the same block risks, so
// X_h <= 2^40 (E_h (1 + 2^-10) + (P + 1) 2^-39) with a wide margin for the
// float roundings on both sides (about 1e-6 relative); when that bound is
// below E_tau for every head the exact test could only answer "no trigger",
// and the pair skips the block pass.
__global__ void __launch_bounds__(kGateThreads) gate_select_kernel(wc_cache c, GateArgs a, const int64_t* pool_used) {
  __shared__ uint64_t tile[kTile];
  __shared__ uint64_t red[kGateThreads];
  __shared__ float hlse[16];
  __shared__ uint64_t hsum[kGateThreads / 64][16];
  __shared__ int kneed;
  const int b = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  if (b == 0 && g == 0 && t == 0) *a.pool_old = *pool_used;
  const int hkv = c.num_kv_heads;
  const int S = a.ctx_len[b];
  const int P = (S + 15) >> 4;
  const int G = a.G;
  const int64_t row0 = ((int64_t)b * a.Hq + g * G) * a.max_pages;   // head n's row: row0 + n * max_pages
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
  const int32_t* eslot = c.exact_slot + (int64_t)a.layer * c.num_pages * hkv + g;   // [phys * hkv]
  if (a.meter && !a.fx) {
    bool quiet = true;
    for (int n = 0; n < G; ++n) {
      const float R = a.meter[b * a.Hq + g * G + n];
      const float E = 2.0f * R / (sqrtf(1.0f + 2.0f * R) + 1.0f);
      quiet = quiet && R >= 0.0f && E * 1.0009765625f + (float)(P + 1) * 1.8189894035458565e-12f <= a.e_tau;
    }
    if (quiet || P == 0) {
      if (t == 0) a.count[b * hkv + g] = 0;
      return;
    }
  }
  // X_h = sum_j rho_fx[h][j] over blocks j = t, t + 256, ...: each round
  // issues its block-risk loads and its repaired-flag gathers together
  uint64_t xs[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) xs[n] = 0;
  float hl[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) hl[n] = n < G ? a.lse[b * a.Hq + g * G + n] : 0.0f;
  const int jend = a.fx ? a.max_pages : P;           // the optional copy covers every block
  for (int j0 = 0; j0 < jend; j0 += 4 * kGateThreads) {
    float lr[4][16];
    int ph[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(j0 + u * kGateThreads + t, a.max_pages - 1);
      ph[u] = ptab[min(j, max(P - 1, 0))];
#pragma unroll
      for (int n = 0; n < 16; ++n) lr[u][n] = n < G ? a.logrisk[row0 + (int64_t)n * a.max_pages + j] : -INFINITY;
    }
    bool live[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kGateThreads + t;
      // repaired blocks (exact keys in the pool) carry no risk
      live[u] = j < P && eslot[(int64_t)ph[u] * hkv] < 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kGateThreads + t;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        if (n < G) {
          const uint64_t v = live[u] ? risk_fx(lr[u][n], hl[n]) : 0;
          xs[n] += v;
          if (a.fx && j < a.max_pages) a.fx[row0 + (int64_t)n * a.max_pages + j] = v;
        }
      }
    }
  }
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    if (n < G) {
      const uint64_t v = wave_sum_u64(xs[n]);
      if ((t & 63) == 0) hsum[t >> 6][n] = v;
    }
  }
  __syncthreads();
  // the trigger test is uniform across the workgroup
  uint64_t xmax = 0;
  for (int n = 0; n < G; ++n) {
    uint64_t X = 0;
    for (int w = 0; w < kGateThreads / 64; ++w) X += hsum[w][n];
    xmax = X > xmax ? X : xmax;
  }
  if (t == 0) a.count[b * hkv + g] = 0;
  if (xmax <= a.T || P == 0) return;

  if (t < 16) hlse[t] = t < G ? a.lse[b * a.Hq + g * G + t] : 0.0f;
  __syncthreads();
  // sort key: max_h rho_fx (at most 2^47) << 16 | (65535 - j): descending =
  // risk descending, ties to the lower block index; non-candidates (repaired
  // or riskless blocks) are 0 and sort last.
  auto key_of = [&](int j) -> uint64_t {
    if (eslot[(int64_t)ptab[j] * hkv] >= 0) return 0;
    uint64_t m = 0;
    for (int n = 0; n < G; ++n) {
      const uint64_t v = risk_fx(a.logrisk[row0 + (int64_t)n * a.max_pages + j], hlse[n]);
      m = v > m ? v : m;
    }
    return m ? (m << 16) | (uint64_t)(65535 - j) : 0;
  };
  const int64_t pair = ((int64_t)b * hkv + g) * a.max_pages;
  const uint64_t* keys = sort_keys(P, tile, a.keys + pair, a.keys2 + pair, t, key_of);
  // a candidate's block and its fixed-point risk for head n (candidates are
  // never repaired)
  auto fx_at = [&](int n, uint64_t k) -> uint64_t {
    const int j = 65535 - (int)(k & 0xFFFF);
    return risk_fx(a.logrisk[row0 + (int64_t)n * a.max_pages + j], hlse[n]);
  };
  // shortest prefix: per head, k_h = #{i : exclusive prefix sum < X_h - T}
  if (t == 0) kneed = 0;
  __syncthreads();
  const int per = (P + kGateThreads - 1) / kGateThreads;
  const int i0 = min(P, t * per), i1 = min(P, i0 + per);
  for (int n = 0; n < G; ++n) {
    uint64_t mine = 0;
    for (int i = i0; i < i1; ++i) {
      const uint64_t k = keys[i];
      if (k) mine += fx_at(n, k);
    }
    // exclusive scan of the per-thread sums (Hillis-Steele in LDS)
    red[t] = mine;
    __syncthreads();
    for (int s = 1; s < kGateThreads; s <<= 1) {
      const uint64_t add = t >= s ? red[t - s] : 0;
      __syncthreads();
      red[t] += add;
      __syncthreads();
    }
    const uint64_t total = red[kGateThreads - 1];
    uint64_t pre = red[t] - mine;
    __syncthreads();
    const uint64_t need = total > a.T ? total - a.T : 0;
    int cnt = 0;
    for (int i = i0; i < i1; ++i) {
      const uint64_t k = keys[i];
      if (!k) break;
      if (pre < need) ++cnt;
      pre += fx_at(n, k);
    }
    red[t] = (uint64_t)cnt;
    __syncthreads();
    for (int s = kGateThreads / 2; s > 0; s >>= 1) {
      if (t < s) red[t] += red[t + s];
      __syncthreads();
    }
    if (t == 0) kneed = max(kneed, (int)red[0]);
    __syncthreads();
  }
  int k = kneed;
  if (a.budget >= 0 && k > a.budget) k = (int)a.budget;
  for (int i = t; i < k; i += kGateThreads) a.sel[pair + i] = 65535 - (int)(keys[i] & 0xFFFF);
  if (t == 0) a.count[b * hkv + g] = k;
}

// Tanh gate selection, one workgroup per (sequence, KV head): candidates are
// the unrepaired blocks with max_h cmax[h][j] > c* (float32 comparison); sort
// key = the float's bits (monotone for values >= 0) << 16 | (65535 - j).
__global__ void __launch_bounds__(kGateThreads) gate_tanh_select_kernel(wc_cache c, GateArgs a, const float* cmax,
                                                                        float cstar, const int64_t* pool_used) {
  __shared__ uint64_t tile[kTile];
  __shared__ int ncand[kGateThreads];
  const int b = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  if (b == 0 && g == 0 && t == 0) *a.pool_old = *pool_used;
  const int hkv = c.num_kv_heads;
  const int P = (a.ctx_len[b] + 15) >> 4;
  const int G = a.G;
  const int64_t row0 = ((int64_t)b * a.Hq + g * G) * a.max_pages;
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
  const int32_t* eslot = c.exact_slot + (int64_t)a.layer * c.num_pages * hkv + g;
  auto key_of = [&](int j) -> uint64_t {
    if (eslot[(int64_t)ptab[j] * hkv] >= 0) return 0;
    float m = 0.0f;
    for (int n = 0; n < G; ++n) m = fmaxf(m, cmax[row0 + (int64_t)n * a.max_pages + j]);
    return m > cstar ? ((uint64_t)__float_as_uint(m) << 16) | (uint64_t)(65535 - j) : 0;
  };
  int mine = 0;
  for (int j = t; j < P; j += kGateThreads) mine += key_of(j) != 0;
  ncand[t] = mine;
  __syncthreads();
  for (int s2 = kGateThreads / 2; s2 > 0; s2 >>= 1) {
    if (t < s2) ncand[t] += ncand[t + s2];
    __syncthreads();
  }
  int k = ncand[0];
  if (t == 0) a.count[b * hkv + g] = 0;
  if (k == 0) return;
  const int64_t pair = ((int64_t)b * hkv + g) * a.max_pages;
  const uint64_t* keys = sort_keys(P, tile, a.keys + pair, a.keys2 + pair, t, key_of);
  if (a.budget >= 0 && k > a.budget) k = (int)a.budget;
  for (int i = t; i < k; i += kGateThreads) a.sel[pair + i] = 65535 - (int)(keys[i] & 0xFFFF);
  if (t == 0) a.count[b * hkv + g] = k;
}

// Pool slots and page-in, one workgroup per ((sequence, KV head) pair bg,
// copy lane y).  Slots go in (b, g, rank) order from the counter's value
// before the call: pair bg starts after the counts of pairs 0 .. bg-1, and
// the selection stops where the pool is full.  One block per workgroup and
// round, 256 threads x 8 bf16.
__global__ void __launch_bounds__(256) gate_copy_kernel(wc_cache c, GateArgs a, const uint16_t* __restrict__ host_k,
                                                        int n_bg, int64_t capacity, int64_t* pool_used,
                                                        int64_t* bytes_paged, int32_t* selected) {
  __shared__ int64_t red[2][4];
  const int bg = blockIdx.x;
  const int hkv = c.num_kv_heads;
  const int b = bg / hkv, g = bg % hkv;
  const int t = threadIdx.x;
  // exclusive prefix of the counts before bg, and their total
  int64_t before = 0, total = 0;
  for (int i = t; i < n_bg; i += 256) {
    const int64_t n = a.count[i];
    total += n;
    before += i < bg ? n : 0;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    before += __shfl_xor(before, m, 64);
    total += __shfl_xor(total, m, 64);
  }
  if ((t & 63) == 0) {
    red[0][t >> 6] = before;
    red[1][t >> 6] = total;
  }
  __syncthreads();
  before = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  total = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const int64_t used0 = *a.pool_old;
  const int64_t start = used0 + before;
  const int64_t cnt = a.count[bg];
  const int64_t room = capacity - start > 0 ? capacity - start : 0;
  const int tk = (int)(cnt < room ? cnt : room);
  if (blockIdx.y == 0) {
    if (bg == n_bg - 1 && t == 0) {
      const int64_t carry = used0 + total;
      const int64_t newu = carry < capacity ? carry : (used0 > capacity ? used0 : capacity);
      *pool_used = newu;
      *bytes_paged += (newu - used0) * 4096;
    }
    if (selected) {
      int32_t* out = selected + (int64_t)bg * (a.max_pages + 1);
      if (t == 0) out[0] = tk;
      for (int j = t; j < tk; j += 256) out[1 + j] = a.sel[(int64_t)bg * a.max_pages + j];
    }
  }
  const int tok = t >> 4, part = t & 15;
  for (int i = blockIdx.y; i < tk; i += gridDim.y) {
    const int j = a.sel[(int64_t)bg * a.max_pages + i];
    const int phys = a.page_table[(int64_t)b * a.max_pages + j];
    const int64_t pg = ((int64_t)a.layer * c.num_pages + phys) * hkv + g;
    const int64_t slot = start + i;
    // the exact bf16 keys go to the pool as they are: [slot][token][128]
    const uint4 v = *reinterpret_cast<const uint4*>(host_k + (pg * 16 + tok) * 128 + 8 * part);
    *reinterpret_cast<uint4*>(c.exact_pool + (slot * 16 + tok) * 128 + 8 * part) = v;
    if (part < 8) c.witness[(pg * 16 + tok) * 8 + part] = 0.0f;
    __syncthreads();
    if (t == 0) c.exact_slot[pg] = (int32_t)slot;
  }
}

// Scratch of wc_gate_pagein_noalloc: the workspace of wc_gate_pagein in a
// file-scope device array (one copy per GPU, held until the process ends).
constexpr size_t kScratchBytes = WC_GATE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

}  // namespace wc

using namespace wc;

namespace {
size_t gate_ws_head(int B, int Hkv, int max_pages) {
  // selected block indices and the count per (sequence, KV head), then the
  // pool counter's value before the call (8-byte aligned)
  const size_t head = (size_t)B * Hkv * max_pages * 4 + (size_t)B * Hkv * 4;
  return ((head + 7) & ~(size_t)7) + 8;
}
}  // namespace

extern "C" size_t wc_gate_workspace_bytes(int B, int Hkv, int max_pages) {
  if (B < 0 || Hkv < 0 || max_pages < 0) return 0;
  // ... and the two sort buffers of 64-bit keys
  return gate_ws_head(B, Hkv, max_pages) + 2 * (size_t)B * Hkv * max_pages * 8;
}

namespace {
// Checks shared by both gates; fills the workspace carve-up.
int gate_prepare(const char* fn, const wc_cache* cache, int layer, int B, int Hq, int max_pages,
                 const void* host_exact_k, void* workspace, size_t ws_bytes, void** dev_host, GateArgs& a) {
  const wc_cache& c = *cache;
  if (c.head_dim != 128 || c.page_size != 16 || c.num_kv_heads < 1 || c.num_bands != 8) {
    set_error("%s: need head_dim 128, 8 bands, 16-token pages", fn);
    return WC_EUNSUPPORTED;
  }
  if (!c.exact_slot || !c.exact_pool || !c.witness || c.pool_capacity < 0) {
    set_error("%s: cache needs exact_slot, exact_pool and witness", fn);
    return WC_EINVAL;
  }
  if (B < 0 || Hq < 1 || Hq % c.num_kv_heads != 0 || Hq / c.num_kv_heads > 16 || max_pages < 1 ||
      max_pages > kMaxPages || layer < 0 || layer >= c.num_layers) {
    set_error("%s: bad B/Hq/max_pages (<= %d)/layer", fn, kMaxPages);
    return WC_EINVAL;
  }
  if (B == 0) return WC_OK;                    // nothing to do (the caller returns too)
  if (ws_bytes < wc_gate_workspace_bytes(B, c.num_kv_heads, max_pages)) {
    set_error("%s: workspace too small", fn);
    return WC_EWORKSPACE;
  }
  // host store: the device view of the pinned allocation; a pointer the
  // device cannot map (pageable memory) is refused before any launch
  *dev_host = nullptr;
  if (hipHostGetDevicePointer(dev_host, const_cast<void*>(host_exact_k), 0) != hipSuccess || !*dev_host) {
    (void)hipGetLastError();
    set_error("%s: host_exact_k is not pinned, device-readable host memory", fn);
    return WC_EINVAL;
  }
  const int hkv = c.num_kv_heads;
  char* ws = (char*)workspace;
  a.sel = (int32_t*)ws;
  ws += (size_t)B * hkv * max_pages * 4;
  a.count = (int32_t*)ws;
  const size_t head = gate_ws_head(B, hkv, max_pages);
  a.pool_old = (int64_t*)((char*)workspace + head - 8);
  a.keys = (uint64_t*)((char*)workspace + head);
  a.keys2 = a.keys + (size_t)B * hkv * max_pages;
  a.B = B;
  a.Hq = Hq;
  a.G = Hq / hkv;
  a.max_pages = max_pages;
  a.layer = layer;
  return WC_OK;
}
}  // namespace

extern "C" int wc_gate_pagein_tanh(const wc_cache* cache, int layer, const float* block_cmax, int B, int Hq,
                                   const int32_t* page_table, int max_pages, const int32_t* ctx_len, double tau,
                                   int64_t budget_blocks, const uint16_t* host_exact_k, int64_t* pool_used,
                                   int64_t* bytes_paged, int32_t* selected, void* workspace, size_t ws_bytes,
                                   void* stream) {
  if (!cache || (B != 0 && (!block_cmax || !page_table || !ctx_len || !host_exact_k || !pool_used || !bytes_paged ||
                             !workspace))) {
    set_error("wc_gate_pagein_tanh: null pointer");
    return WC_EINVAL;
  }
  if (!(tau >= 0.0)) {
    set_error("wc_gate_pagein_tanh: need tau >= 0");
    return WC_EINVAL;
  }
  GateArgs a{};
  void* dev_host = nullptr;
  if (int e = gate_prepare("wc_gate_pagein_tanh", cache, layer, B, Hq, max_pages, host_exact_k, workspace, ws_bytes,
                           &dev_host, a))
    return e;
  if (B == 0) return WC_OK;
  const wc_cache& c = *cache;
  a.page_table = page_table;
  a.ctx_len = ctx_len;
  a.budget = budget_blocks;
  const float cstar = tau >= 1.0 ? INFINITY : (float)(2.0 * atanh(tau));
  const int hkv = c.num_kv_heads;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(gate_tanh_select_kernel, dim3((unsigned)B, (unsigned)hkv), dim3(kGateThreads), 0, st, c, a,
                     block_cmax, cstar, (const int64_t*)pool_used);
  if (int e = check_launch("wc_gate_pagein_tanh select")) return e;
  hipLaunchKernelGGL(gate_copy_kernel, dim3((unsigned)(B * hkv), 8u), dim3(256), 0, st, c, a,
                     (const uint16_t*)dev_host, B * hkv, c.pool_capacity, pool_used, bytes_paged, selected);
  return check_launch("wc_gate_pagein_tanh copy");
}

namespace {
int gate_pagein(const char* fn, const wc_cache* cache, int layer, const float* block_logrisk, const float* lse,
                const float* meter, int B, int Hq, const int32_t* page_table, int max_pages, const int32_t* ctx_len,
                double tau, int64_t budget_blocks, const uint16_t* host_exact_k, int64_t* pool_used,
                int64_t* bytes_paged, int32_t* selected, uint64_t* rho_fx, void* workspace, size_t ws_bytes,
                void* stream) {
  if (!cache || (B != 0 && (!block_logrisk || !lse || !page_table || !ctx_len || !host_exact_k || !pool_used ||
                             !bytes_paged || !workspace))) {
    set_error("%s: null pointer", fn);
    return WC_EINVAL;
  }
  const double et = sqrt(1.0 + 2.0 * tau) - 1.0;
  if (!(tau >= 0.0) || !(et < 64.0)) {
    set_error("%s: need 0 <= tau and sqrt(1 + 2 tau) - 1 < 64", fn);
    return WC_EINVAL;
  }
  GateArgs a{};
  void* dev_host = nullptr;
  if (int e = gate_prepare(fn, cache, layer, B, Hq, max_pages, host_exact_k, workspace, ws_bytes, &dev_host, a))
    return e;
  if (B == 0) return WC_OK;
  const wc_cache& c = *cache;
  const int hkv = c.num_kv_heads;
  a.logrisk = block_logrisk;
  a.lse = lse;
  a.meter = meter;
  // E_tau rounded down to float: the quiet test errs toward the exact pass
  a.e_tau = nextafterf((float)et, 0.0f);
  a.page_table = page_table;
  a.ctx_len = ctx_len;
  a.fx = rho_fx;
  a.T = (uint64_t)floor(et * 1099511627776.0);
  a.budget = budget_blocks;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(gate_select_kernel, dim3((unsigned)B, (unsigned)hkv), dim3(kGateThreads), 0, st, c, a,
                     (const int64_t*)pool_used);
  if (int e = check_launch(fn)) return e;
  hipLaunchKernelGGL(gate_copy_kernel, dim3((unsigned)(B * hkv), 8u), dim3(256), 0, st, c, a,
                     (const uint16_t*)dev_host, B * hkv, c.pool_capacity, pool_used, bytes_paged, selected);
  return check_launch(fn);
}

// The device address of `scratch` on each device, looked up once per device
// (with that device current) on its first use.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_ptr(const char* fn, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    set_error("%s: no current HIP device", fn);
    return WC_EHIP;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      set_error("%s: hipGetSymbolAddress of the scratch array failed: %s", fn, hipGetErrorString(e));
      return WC_EHIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return WC_OK;
}
}  // namespace

extern "C" int wc_gate_pagein(const wc_cache* cache, int layer, const float* block_logrisk, const float* lse,
                              const float* meter, int B, int Hq, const int32_t* page_table, int max_pages,
                              const int32_t* ctx_len, double tau, int64_t budget_blocks, const uint16_t* host_exact_k,
                              int64_t* pool_used, int64_t* bytes_paged, int32_t* selected, uint64_t* rho_fx,
                              void* workspace, size_t ws_bytes, void* stream) {
  return gate_pagein("wc_gate_pagein", cache, layer, block_logrisk, lse, meter, B, Hq, page_table, max_pages, ctx_len,
                     tau, budget_blocks, host_exact_k, pool_used, bytes_paged, selected, rho_fx, workspace, ws_bytes,
                     stream);
}

extern "C" int wc_gate_pagein_noalloc(const wc_cache* cache, int layer, const float* block_logrisk, const float* lse,
                                      const float* meter, int B, int Hq, const int32_t* page_table, int max_pages,
                                      const int32_t* ctx_len, double tau, int64_t budget_blocks,
                                      const uint16_t* host_exact_k, int64_t* pool_used, int64_t* bytes_paged,
                                      int32_t* selected, uint64_t* rho_fx, void* stream) {
  const char* fn = "wc_gate_pagein_noalloc";
  if (!cache) {
    set_error("%s: null pointer", fn);
    return WC_EINVAL;
  }
  if (B < 0 || max_pages < 0 || cache->num_kv_heads < 1) {
    set_error("%s: bad B/max_pages/num_kv_heads", fn);
    return WC_EINVAL;
  }
  const size_t need = wc_gate_workspace_bytes(B, cache->num_kv_heads, max_pages);
  if (need > kScratchBytes) {
    set_error("%s: needs %zu bytes of scratch for B=%d, Hkv=%d, max_pages=%d; the static scratch holds %zu", fn,
              need, B, cache->num_kv_heads, max_pages, kScratchBytes);
    return WC_EWORKSPACE;
  }
  void* ws = nullptr;
  if (B != 0) {
    if (int e = scratch_ptr(fn, &ws)) return e;
  }
  return gate_pagein(fn, cache, layer, block_logrisk, lse, meter, B, Hq, page_table, max_pages, ctx_len, tau,
                     budget_blocks, host_exact_k, pool_used, bytes_paged, selected, rho_fx, ws, kScratchBytes,
                     stream);
}
