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
// Kernels: (1) per (sequence, KV head, 256-block chunk): fixed-point risks
// of all the group's query heads and their chunk sums; (2) per (sequence, KV
// head): trigger test on the sums, then (rarely) bitonic sort of the
// candidates by risk in LDS and per-head scans for the shortest sufficient
// prefix; (3) one workgroup: exclusive scan of the counts in (sequence, head)
// order hands out exact-pool slots deterministically; (4) copy each selected
// block from pinned host memory (zero-copy reads), store it as fp16 with a
// per-token power of two, zero its witness, mark it.
//
// The tanh gate (the page-in comparison of the summary): the bound
// tanh(max_t c_t / 2) is <= tau for every head exactly when no unrepaired
// token has c_t > c* = 2 artanh(tau), so kernel (2) is replaced by one that
// takes every unrepaired block whose largest bound over the group's heads
// exceeds c*, ranked by that bound; (3) and (4) are shared.
#include <math.h>

#include "wc_common.h"

namespace wc {

constexpr int kFxBits = 40;
constexpr uint64_t kFxCap = uint64_t(1) << 47;
constexpr int kMaxSortPages = 4096;

struct GateArgs {
  const float* logrisk;
  const float* lse;
  const int32_t* page_table;
  const int32_t* ctx_len;
  uint64_t* fx;           // [B][Hq][max_pages], optional copy for the caller
  uint64_t* xpart;        // [B][Hq][nchunk]: per 256-block chunk sums of rho_fx
  int32_t* sel;           // [B][Hkv][max_pages]
  int32_t* count;         // [B][Hkv]
  int32_t* base;          // [B][Hkv]
  int32_t* take;          // [B][Hkv]
  int B, Hq, G, max_pages, layer, nchunk;
  uint64_t T;
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

// Fixed-point risks of one 256-block chunk of one (sequence, KV head), all
// its query heads: chunk sums for the trigger test (and the optional copy).
__global__ void __launch_bounds__(256) gate_risk_kernel(wc_cache c, GateArgs a) {
  __shared__ uint64_t wsum[4][16];
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int hkv = c.num_kv_heads;
  const int P = (a.ctx_len[b] + 15) >> 4;
  const int G = a.G;
  const int j = chunk * 256 + t;
  const int64_t row0 = ((int64_t)b * a.Hq + g * G) * a.max_pages;
  // every load is issued unconditionally (indices clamped into range) so that
  // they are all in flight together
  const int jc = min(j, a.max_pages - 1);
  float lr[16], ls[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const int nc = min(n, G - 1);
    lr[n] = a.logrisk[row0 + (int64_t)nc * a.max_pages + jc];
    ls[n] = a.lse[b * a.Hq + g * G + nc];
  }
  const int phys = a.page_table[(int64_t)b * a.max_pages + min(j, max(P - 1, 0))];
  // repaired blocks (exact keys in the pool) carry no risk
  const bool live = j < P && c.exact_slot[((int64_t)a.layer * c.num_pages + phys) * hkv + g] < 0;
  uint64_t part[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) part[n] = (n < G && live) ? risk_fx(lr[n], ls[n]) : 0;
  if (a.fx && j < a.max_pages) {
#pragma unroll
    for (int n = 0; n < 16; ++n)
      if (n < G) a.fx[row0 + (int64_t)n * a.max_pages + j] = part[n];
  }
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    if (n < G) {
      const uint64_t v = wave_sum_u64(part[n]);
      if ((t & 63) == 0) wsum[t >> 6][n] = v;
    }
  }
  __syncthreads();
  if (t < G)
    a.xpart[((int64_t)b * a.Hq + g * G + t) * a.nchunk + chunk] = wsum[0][t] + wsum[1][t] + wsum[2][t] + wsum[3][t];
}

// Bitonic sort of keys[0 .. np2) (np2 a power of two) in LDS, descending;
// 256 threads, every thread calls it.
__device__ void sort_desc(uint64_t* keys, int np2, int t) {
  for (int kk = 2; kk <= np2; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = t; i < np2; i += 256) {
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

__global__ void __launch_bounds__(256) gate_select_kernel(wc_cache c, GateArgs a) {
  __shared__ uint64_t keys[kMaxSortPages];
  __shared__ uint64_t red[256];
  __shared__ float hlse[16];
  __shared__ uint8_t rep[kMaxSortPages];
  __shared__ int kneed;
  const int b = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int hkv = c.num_kv_heads;
  const int S = a.ctx_len[b];
  const int P = (S + 15) >> 4;
  const int G = a.G;
  const int64_t row0 = ((int64_t)b * a.Hq + g * G) * a.max_pages;   // head n's row: row0 + n * max_pages
  // X_h from the chunk sums; the trigger test is uniform across the workgroup
  uint64_t xmax = 0;
  for (int n = 0; n < G; ++n) {
    uint64_t X = 0;
    for (int k = 0; k < a.nchunk; ++k) X += a.xpart[((int64_t)b * a.Hq + g * G + n) * a.nchunk + k];
    xmax = X > xmax ? X : xmax;
  }
  if (t == 0) a.count[b * hkv + g] = 0;
  if (xmax <= a.T || P == 0) return;

  if (t < 16) hlse[t] = t < G ? a.lse[b * a.Hq + g * G + t] : 0.0f;
  for (int j = t; j < P; j += 256) {
    const int phys = a.page_table[(int64_t)b * a.max_pages + j];
    rep[j] = c.exact_slot[((int64_t)a.layer * c.num_pages + phys) * hkv + g] >= 0;
  }
  __syncthreads();
  auto fx_of = [&](int n, int j) -> uint64_t {
    return rep[j] ? 0 : risk_fx(a.logrisk[row0 + (int64_t)n * a.max_pages + j], hlse[n]);
  };

  // sort key: max_h rho_fx (47 bits) << 16 | (65535 - j): descending = risk
  // descending, ties to the lower block index; non-candidates are 0.
  int np2 = 1;
  while (np2 < P) np2 <<= 1;
  for (int j = t; j < np2; j += 256) {
    uint64_t k = 0;
    if (j < P) {
      uint64_t m = 0;
      for (int n = 0; n < G; ++n) {
        const uint64_t v = fx_of(n, j);
        m = v > m ? v : m;
      }
      k = m ? (m << 16) | (uint64_t)(65535 - j) : 0;
    }
    keys[j] = k;
  }
  __syncthreads();
  sort_desc(keys, np2, t);
  // shortest prefix: per head, k_h = #{i : exclusive prefix sum < X_h - T}
  if (t == 0) kneed = 0;
  __syncthreads();
  const int per = (P + 255) / 256;
  const int i0 = t * per, i1 = min(P, i0 + per);
  for (int n = 0; n < G; ++n) {
    uint64_t mine = 0;
    for (int i = i0; i < i1; ++i) {
      const uint64_t k = keys[i];
      if (k) mine += fx_of(n, 65535 - (int)(k & 0xFFFF));
    }
    // exclusive scan of the per-thread sums (Hillis-Steele in LDS)
    red[t] = mine;
    __syncthreads();
    for (int s = 1; s < 256; s <<= 1) {
      const uint64_t add = t >= s ? red[t - s] : 0;
      __syncthreads();
      red[t] += add;
      __syncthreads();
    }
    const uint64_t total = red[255];
    uint64_t pre = red[t] - mine;
    __syncthreads();
    const uint64_t need = total > a.T ? total - a.T : 0;
    int cnt = 0;
    for (int i = i0; i < i1; ++i) {
      const uint64_t k = keys[i];
      if (!k) break;
      if (pre < need) ++cnt;
      pre += fx_of(n, 65535 - (int)(k & 0xFFFF));
    }
    red[t] = (uint64_t)cnt;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (t < s) red[t] += red[t + s];
      __syncthreads();
    }
    if (t == 0) kneed = max(kneed, (int)red[0]);
    __syncthreads();
  }
  int k = kneed;
  if (a.budget >= 0 && k > a.budget) k = (int)a.budget;
  for (int i = t; i < k; i += 256) a.sel[((int64_t)b * hkv + g) * a.max_pages + i] = 65535 - (int)(keys[i] & 0xFFFF);
  if (t == 0) a.count[b * hkv + g] = k;
}

// Tanh gate selection, one workgroup per (sequence, KV head): candidates are
// the unrepaired blocks with max_h cmax[h][j] > c* (float32 comparison); sort
// key = the float's bits (monotone for values >= 0) << 16 | (65535 - j).
__global__ void __launch_bounds__(256) gate_tanh_select_kernel(wc_cache c, GateArgs a, const float* cmax,
                                                               float cstar) {
  __shared__ uint64_t keys[kMaxSortPages];
  __shared__ int ncand[256];
  const int b = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int hkv = c.num_kv_heads;
  const int P = (a.ctx_len[b] + 15) >> 4;
  const int G = a.G;
  const int64_t row0 = ((int64_t)b * a.Hq + g * G) * a.max_pages;
  int np2 = 1;
  while (np2 < P) np2 <<= 1;
  int mine = 0;
  for (int j = t; j < np2; j += 256) {
    uint64_t k = 0;
    if (j < P) {
      const int phys = a.page_table[(int64_t)b * a.max_pages + j];
      if (c.exact_slot[((int64_t)a.layer * c.num_pages + phys) * hkv + g] < 0) {
        float m = 0.0f;
        for (int n = 0; n < G; ++n) m = fmaxf(m, cmax[row0 + (int64_t)n * a.max_pages + j]);
        if (m > cstar) {
          k = ((uint64_t)__float_as_uint(m) << 16) | (uint64_t)(65535 - j);
          ++mine;
        }
      }
    }
    keys[j] = k;
  }
  ncand[t] = mine;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (t < s2) ncand[t] += ncand[t + s2];
    __syncthreads();
  }
  int k = ncand[0];
  if (k > 0) sort_desc(keys, np2, t);
  if (a.budget >= 0 && k > a.budget) k = (int)a.budget;
  for (int i = t; i < k; i += 256) a.sel[((int64_t)b * hkv + g) * a.max_pages + i] = 65535 - (int)(keys[i] & 0xFFFF);
  if (t == 0) a.count[b * hkv + g] = k;
}

// One workgroup: slots in (b, g, rank) order from *pool_used, stop at capacity.
__global__ void __launch_bounds__(256) gate_assign_kernel(GateArgs a, int n_bg, int64_t capacity, int64_t* pool_used,
                                                          int64_t* bytes_paged, int32_t* selected) {
  __shared__ int64_t sc[256];
  __shared__ int64_t carry;
  const int t = threadIdx.x;
  if (t == 0) carry = *pool_used;
  __syncthreads();
  for (int c0 = 0; c0 < n_bg; c0 += 256) {
    const int i = c0 + t;
    const int64_t cnt = i < n_bg ? a.count[i] : 0;
    sc[t] = cnt;
    __syncthreads();
    for (int s = 1; s < 256; s <<= 1) {
      const int64_t add = t >= s ? sc[t - s] : 0;
      __syncthreads();
      sc[t] += add;
      __syncthreads();
    }
    const int64_t start = carry + sc[t] - cnt;
    if (i < n_bg) {
      int64_t room = capacity - start;
      room = room < 0 ? 0 : room;
      const int64_t tk = cnt < room ? cnt : room;
      a.base[i] = (int32_t)start;
      a.take[i] = (int32_t)tk;
    }
    __syncthreads();
    if (t == 255) carry += sc[255];
    __syncthreads();
  }
  if (t == 0) {
    const int64_t used0 = *pool_used;
    const int64_t newu = carry < capacity ? carry : (used0 > capacity ? used0 : capacity);
    *pool_used = newu;
    *bytes_paged += (newu - used0) * 4096;
  }
  if (selected) {
    for (int i = 0; i < n_bg; ++i) {
      int32_t* out = selected + (int64_t)i * (a.max_pages + 1);
      const int tk = a.take[i];
      if (t == 0) out[0] = tk;
      for (int j = t; j < tk; j += 256) out[1 + j] = a.sel[(int64_t)i * a.max_pages + j];
    }
  }
}

// Copy selected blocks: one workgroup per block, 256 threads x 8 bf16.
__global__ void __launch_bounds__(256) gate_copy_kernel(wc_cache c, GateArgs a, const uint16_t* __restrict__ host_k) {
  const int bg = blockIdx.x;
  const int hkv = c.num_kv_heads;
  const int b = bg / hkv, g = bg % hkv;
  const int tk = a.take[bg];
  const int t = threadIdx.x;
  const int tok = t >> 4, part = t & 15;
  for (int i = blockIdx.y; i < tk; i += gridDim.y) {
    const int j = a.sel[(int64_t)bg * a.max_pages + i];
    const int phys = a.page_table[(int64_t)b * a.max_pages + j];
    const int64_t pg = ((int64_t)a.layer * c.num_pages + phys) * hkv + g;
    const int64_t slot = (int64_t)a.base[bg] + i;
    const uint4 v = *reinterpret_cast<const uint4*>(host_k + (pg * 16 + tok) * 128 + 8 * part);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float x[8];
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      am = fmaxf(am, fmaxf(fabsf(x[2 * e]), fabsf(x[2 * e + 1])));
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) am = fmaxf(am, __shfl_xor(am, m, 64));
    int ex = 0, sh = 0;
    if (am > 0.0f && am < INFINITY) {
      frexpf(am, &ex);
      sh = 15 - ex;                            // row max in [2^14, 2^15)
    }
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      _Float16 h0 = (_Float16)ldexpf(x[2 * e], sh), h1 = (_Float16)ldexpf(x[2 * e + 1], sh);
      o[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    }
    *reinterpret_cast<uint4*>(c.exact_pool + (slot * 16 + tok) * 128 + 8 * part) = make_uint4(o[0], o[1], o[2], o[3]);
    if (part == 0) c.exact_scale[slot * 16 + tok] = ldexpf(1.0f, -sh);
    if (part < 8) c.witness[(pg * 16 + tok) * 8 + part] = 0.0f;
    __syncthreads();
    if (t == 0) c.exact_slot[pg] = (int32_t)slot;
  }
}

}  // namespace wc

using namespace wc;

extern "C" size_t wc_gate_workspace_bytes(int B, int Hkv, int max_pages) {
  if (B < 0 || Hkv < 0 || max_pages < 0) return 0;
  // chunk sums (up to 16 query heads per KV head), selected block indices,
  // then count / base / take per (sequence, KV head)
  const size_t nchunk = ((size_t)max_pages + 255) / 256;
  return (size_t)B * Hkv * 16 * nchunk * 8 + (size_t)B * Hkv * max_pages * 4 + (size_t)B * Hkv * 3 * 4;
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
  if (!c.exact_slot || !c.exact_pool || !c.exact_scale || !c.witness || c.pool_capacity < 0) {
    set_error("%s: cache needs exact_slot, exact_pool, exact_scale and witness", fn);
    return WC_EINVAL;
  }
  if (B < 0 || Hq < 1 || Hq % c.num_kv_heads != 0 || Hq / c.num_kv_heads > 16 || max_pages < 1 ||
      max_pages > kMaxSortPages || layer < 0 || layer >= c.num_layers) {
    set_error("%s: bad B/Hq/max_pages (<= %d)/layer", fn, kMaxSortPages);
    return WC_EINVAL;
  }
  if (ws_bytes < wc_gate_workspace_bytes(B, c.num_kv_heads, max_pages)) {
    set_error("%s: workspace too small", fn);
    return WC_EWORKSPACE;
  }
  // host store: translate to the device view of the pinned allocation
  *dev_host = nullptr;
  if (hipHostGetDevicePointer(dev_host, const_cast<void*>(host_exact_k), 0) != hipSuccess || !*dev_host) {
    (void)hipGetLastError();
    *dev_host = const_cast<void*>(host_exact_k);   // unified addressing: same pointer
  }
  const int hkv = c.num_kv_heads;
  char* ws = (char*)workspace;
  const int nchunk = (max_pages + 255) / 256;
  a.xpart = (uint64_t*)ws;
  ws += (size_t)B * hkv * 16 * nchunk * 8;
  a.sel = (int32_t*)ws;
  ws += (size_t)B * hkv * max_pages * 4;
  a.count = (int32_t*)ws;
  a.base = a.count + B * hkv;
  a.take = a.base + B * hkv;
  a.B = B;
  a.Hq = Hq;
  a.G = Hq / hkv;
  a.max_pages = max_pages;
  a.layer = layer;
  a.nchunk = nchunk;
  return WC_OK;
}
}  // namespace

extern "C" int wc_gate_pagein_tanh(const wc_cache* cache, int layer, const float* block_cmax, int B, int Hq,
                                   const int32_t* page_table, int max_pages, const int32_t* ctx_len, double tau,
                                   int64_t budget_blocks, const uint16_t* host_exact_k, int64_t* pool_used,
                                   int64_t* bytes_paged, int32_t* selected, void* workspace, size_t ws_bytes,
                                   void* stream) {
  if (!cache || !block_cmax || !page_table || !ctx_len || !host_exact_k || !pool_used || !bytes_paged ||
      !workspace) {
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
  hipLaunchKernelGGL(gate_tanh_select_kernel, dim3((unsigned)B, (unsigned)hkv), dim3(256), 0, st, c, a, block_cmax,
                     cstar);
  if (int e = check_launch("wc_gate_pagein_tanh select")) return e;
  hipLaunchKernelGGL(gate_assign_kernel, dim3(1), dim3(256), 0, st, a, B * hkv, c.pool_capacity, pool_used,
                     bytes_paged, selected);
  if (int e = check_launch("wc_gate_pagein_tanh assign")) return e;
  hipLaunchKernelGGL(gate_copy_kernel, dim3((unsigned)(B * hkv), 8u), dim3(256), 0, st, c, a,
                     (const uint16_t*)dev_host);
  return check_launch("wc_gate_pagein_tanh copy");
}

extern "C" int wc_gate_pagein(const wc_cache* cache, int layer, const float* block_logrisk, const float* lse, int B,
                              int Hq, const int32_t* page_table, int max_pages, const int32_t* ctx_len, double tau,
                              int64_t budget_blocks, const uint16_t* host_exact_k, int64_t* pool_used,
                              int64_t* bytes_paged, int32_t* selected, uint64_t* rho_fx, void* workspace,
                              size_t ws_bytes, void* stream) {
  if (!cache || !block_logrisk || !lse || !page_table || !ctx_len || !host_exact_k || !pool_used || !bytes_paged ||
      !workspace) {
    set_error("wc_gate_pagein: null pointer");
    return WC_EINVAL;
  }
  const double et = sqrt(1.0 + 2.0 * tau) - 1.0;
  if (!(tau >= 0.0) || !(et < 64.0)) {
    set_error("wc_gate_pagein: need 0 <= tau and sqrt(1 + 2 tau) - 1 < 64");
    return WC_EINVAL;
  }
  GateArgs a{};
  void* dev_host = nullptr;
  if (int e = gate_prepare("wc_gate_pagein", cache, layer, B, Hq, max_pages, host_exact_k, workspace, ws_bytes,
                           &dev_host, a))
    return e;
  if (B == 0) return WC_OK;
  const wc_cache& c = *cache;
  const int hkv = c.num_kv_heads;
  const int nchunk = a.nchunk;
  a.logrisk = block_logrisk;
  a.lse = lse;
  a.page_table = page_table;
  a.ctx_len = ctx_len;
  a.fx = rho_fx;
  a.T = (uint64_t)floor(et * 1099511627776.0);
  a.budget = budget_blocks;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(gate_risk_kernel, dim3((unsigned)nchunk, (unsigned)hkv, (unsigned)B), dim3(256), 0, st, c, a);
  if (int e = check_launch("wc_gate_pagein risk")) return e;
  hipLaunchKernelGGL(gate_select_kernel, dim3((unsigned)B, (unsigned)hkv), dim3(256), 0, st, c, a);
  if (int e = check_launch("wc_gate_pagein select")) return e;
  hipLaunchKernelGGL(gate_assign_kernel, dim3(1), dim3(256), 0, st, a, B * hkv, c.pool_capacity, pool_used,
                     bytes_paged, selected);
  if (int e = check_launch("wc_gate_pagein assign")) return e;
  hipLaunchKernelGGL(gate_copy_kernel, dim3((unsigned)(B * hkv), 8u), dim3(256), 0, st, c, a,
                     (const uint16_t*)dev_host);
  return check_launch("wc_gate_pagein copy");
}
