// Write path: quantize K/V rows and store the key witness.
//
// WitCert summary (Tier B paragraph): subtractive dither
// x^ = s(round(x/s + xi) - xi), xi regenerated at read time; (witness-theorem
// paragraph) w_{t,b} = ||r_{t,b}|| stored once at write time; black-box
// schemes (fp8 raw cast, kivi-2bit) measured through the same witness.
//
// INT8 / fp8: one row = one (layer, token, KV head) of 128 channels, handled
// by 16 lanes with 8 channels each (one 16 B bf16 load), 4 rows per wave.
// The row absmax and the band sums are 16-lane xor-shuffle reductions; band
// b = dims 8b..8b+7 (lane b) and 64+8b..64+8b+7 (lane b+8).
#include <stdarg.h>
#include <stdio.h>

#include <type_traits>

#include "wc_common.h"

namespace wc {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return WC_EHIP;
  }
  return WC_OK;
}

// The same maximum for values that are >= 0 and not NaN: their order is that
// of their bit patterns, one integer max with a DPP operand per step.
__device__ __forceinline__ float row16_max_nonneg(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, kRowRor8, 0xF, 0xF, false));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, kRowRor4, 0xF, 0xF, false));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, kQuadSwap2, 0xF, 0xF, false));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, kQuadSwap1, 0xF, 0xF, false));
  return __uint_as_float(u);
}
// Lane N of each 16-lane row, to every lane of that row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row16_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

// Inputs are read once and code blocks written once: their accesses carry
// the non-temporal cache policy (native vector types, which the builtins take).
typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));
typedef float nt_f4 __attribute__((ext_vector_type(4)));

// One lane's 8 input channels as loaded (16 B of bf16 or 32 B of fp32), kept
// raw so that the loads can be issued ahead of the work that waits on them.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  nt_u4 a;
};
template <>
struct Raw8<float> {
  nt_f4 a, b;
};

template <typename T>
__device__ __forceinline__ Raw8<T> load_raw8(const T* p);
template <>
__device__ __forceinline__ Raw8<float> load_raw8<float>(const float* p) {
  return Raw8<float>{__builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(p)),
                     __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(p + 4))};
}
template <>
__device__ __forceinline__ Raw8<uint16_t> load_raw8<uint16_t>(const uint16_t* p) {
  return Raw8<uint16_t>{__builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p))};
}

__device__ __forceinline__ void unpack8(const Raw8<float>& r, float (&x)[8]) {
  x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
  x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}
__device__ __forceinline__ void unpack8(const Raw8<uint16_t>& r, float (&x)[8]) {
  const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]) {
  unpack8(load_raw8<T>(p), x);
}

struct RowArgs {
  int64_t n_tok;
  int64_t layer_stride;
  int64_t num_pages;
  int hkv;
  int layer0;
  int n_layers;
  const int64_t* slot;
  const int32_t* pos;
  const uint64_t* seed;
};

// Quantize the 8 channels of one lane; returns codes packed little-endian
// in two words (INT8: offset binary code + 128) and the residual r = x^ - x.
// words[w] holds the draws of channels 8 lane16 + 2w (low half) and + 1.
// Bit i of `exact` marks a bypassed channel: code 0, residual 0.
template <int SCHEME>
__device__ __forceinline__ void quant8(const float (&x)[8], float s, float inv, const uint32_t (&words)[4],
                                       uint32_t exact, uint32_t (&packed)[2], float (&r)[8]) {
  packed[0] = packed[1] = 0;
  if (SCHEME == WC_FP8_E4M3) {
    // gfx950's conversions are OCP e4m3fn with round to nearest even; with the
    // input clamped to +-448 first the encoding saturates there (a NaN input
    // takes +-448 by its sign), and the decode is exact
    float xc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xc[i] = fminf(fmaxf(x[i], -448.0f), 448.0f);
      xc[i] = x[i] != x[i] ? copysignf(448.0f, x[i]) : xc[i];
    }
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(xc[0], xc[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(xc[2], xc[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(xc[4], xc[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(xc[6], xc[7], w1, true);
    packed[0] = (uint32_t)w0;
    packed[1] = (uint32_t)w1;
    r[0] = __builtin_amdgcn_cvt_f32_fp8(w0, 0) - x[0];
    r[1] = __builtin_amdgcn_cvt_f32_fp8(w0, 1) - x[1];
    r[2] = __builtin_amdgcn_cvt_f32_fp8(w0, 2) - x[2];
    r[3] = __builtin_amdgcn_cvt_f32_fp8(w0, 3) - x[3];
    r[4] = __builtin_amdgcn_cvt_f32_fp8(w1, 0) - x[4];
    r[5] = __builtin_amdgcn_cvt_f32_fp8(w1, 1) - x[5];
    r[6] = __builtin_amdgcn_cvt_f32_fp8(w1, 2) - x[6];
    r[7] = __builtin_amdgcn_cvt_f32_fp8(w1, 3) - x[7];
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t code;
    float xr;
    if (SCHEME == WC_DITHER_INT8) {
      const uint32_t k16 = (i & 1) ? (words[i >> 1] >> 16) : (words[i >> 1] & 0xFFFFu);
      const float xi = fmaf((float)k16, 1.52587890625e-05f, -0.5f);   // exact
      // an all-zero row has s = inv = 0: y = xi in [-1/2, 1/2) rounds to 0
      // and the residual below is -x = 0, so no case of its own is needed
      const float y = add_rn(mul_rn(x[i], inv), xi);
      float q = __builtin_amdgcn_fmed3f(rintf(y), -128.0f, 127.0f);
      xr = fmaf(s, q - xi, -x[i]);              // q - xi exact; one rounding
      if ((exact >> i) & 1u) {
        q = 0.0f;
        xr = 0.0f;
      }
      code = (uint32_t)((int32_t)q + 128);
    } else if (SCHEME == WC_RTN_INT8) {
      // (s = inv = 0 on an all-zero row gives code 0 and residual 0 as well)
      const float q = __builtin_amdgcn_fmed3f(rintf(mul_rn(x[i], inv)), -128.0f, 127.0f);
      code = (uint32_t)((int32_t)q + 128);
      xr = fmaf(s, q, -x[i]);                   // one rounding
    } else {
      code = 0u;                                // (fp8 returned above)
      xr = 0.0f;
    }
    packed[i >> 2] |= code << (8 * (i & 3));
    r[i] = xr;
  }
}

// One (token, KV head) row, both tensors, on 16 lanes of 8 channels: codes
// (packed little-endian, INT8 as offset binary), row scales, the key's band
// witness (lanes 0..7 hold bands 0..7) and the value witness.
struct RowQ {
  uint32_t kp[2], vp[2];
  float ks, vs, w, wv;
};

// OUTL: dithered INT8 keys with the outlier bypass (bf16 input): the
// channels in omask are excluded from the key absmax, coded 0 with a zero
// residual (their exact keys go to the side store, written by the caller).
//
// The row-level steps are shared out over the row's 16 lanes instead of being
// repeated on each: the four scale quotients (s and 1/s of K and of V) are one
// correctly rounded division, lanes 4j..4j+3 taking quotient j, and the key's
// band norms (lanes 0..7) and the value's row norm (lanes 8..15) one square
// root; each result is then broadcast within the row.
template <typename T, int SCHEME>
__device__ __forceinline__ RowQ quant_row(const Raw8<T>& krow, const Raw8<T>& vrow, const uint32_t (&words)[4],
                                          uint32_t omask) {
  constexpr bool SC = SCHEME == WC_DITHER_INT8 || SCHEME == WC_RTN_INT8;
  const int lane16 = threadIdx.x & 15;
  float xk[8], xv[8];
  unpack8(krow, xk);
  unpack8(vrow, xv);
  float sk = 0.0f, ik = 0.0f, sv = 0.0f, iv = 0.0f;
  if (SC) {
    // absmax from 0 up: a NaN input never wins, so both maxima are finite or
    // +inf and their 16-lane maxima can be taken on the bit patterns
    float amk = 0.0f, amv = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      amk = fmaxf(amk, ((omask >> k) & 1u) ? 0.0f : fabsf(xk[k]));
      amv = fmaxf(amv, fabsf(xv[k]));
    }
    amk = row16_max_nonneg(amk);
    amv = row16_max_nonneg(amv);
    const int role = lane16 >> 2;              // 0: amk / 127, 1: 127 / amk, 2, 3: the same of amv
    const float am = role < 2 ? amk : amv;
    // (operands selected first: one division sequence for the wave, not two
    // divergent ones)
    const float num = (role & 1) ? 127.0f : am, den = (role & 1) ? am : 127.0f;
    const float qt = div_rn(num, den);
    // (an all-zero row keeps s = 1/s = 0)
    sk = amk > 0.0f ? row16_bcast<0>(qt) : 0.0f;
    ik = amk > 0.0f ? row16_bcast<4>(qt) : 0.0f;
    sv = amv > 0.0f ? row16_bcast<8>(qt) : 0.0f;
    iv = amv > 0.0f ? row16_bcast<12>(qt) : 0.0f;
  }
  RowQ o;
  float rk[8], rv[8];
  quant8<SCHEME>(xk, sk, ik, words, omask, o.kp, rk);
  quant8<SCHEME>(xv, sv, iv, words, 0u, o.vp, rv);
  o.ks = sk;
  o.vs = sv;
  float ssk = 0.0f, ssv = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ssk = fmaf(rk[k], rk[k], ssk);
    ssv = fmaf(rv[k], rv[k], ssv);
  }
  ssk += dpp_f<kRowRor8>(ssk);                 // lanes l, l + 8: the two halves of band l % 8
  ssv = row16_sum(ssv);                        // value witness ||v^ - v|| over the row's 128 channels
  const float nrm = sqrtf(lane16 < 8 ? ssk : ssv) * kWitnessGuard;
  o.w = nrm;                                   // (lanes 0..7: band lane16)
  o.wv = row16_bcast<8>(nrm);
  return o;
}

// Bypassed channels among lane16's 8 (bit i = channel 8 lane16 + i), and the
// channel whose exact key lane16 copies into the side store (-1: none).
__device__ __forceinline__ void bypass_lanes(const wc_cache& c, int layer, int hkv, int g, int lane16,
                                             uint32_t& omask, int& ochan) {
  const int m = c.num_outliers;
  const int32_t* oc = c.outlier_ch + ((int64_t)layer * hkv + g) * m;
  omask = 0;
  for (int e = 0; e < m; ++e) {
    const int ch = oc[e];
    omask |= (ch >> 3) == lane16 ? 1u << (ch & 7) : 0u;
  }
  ochan = lane16 < m ? (oc[lane16] & 127) : -1;   // (in range even for a corrupt list)
}

// Persistent repair: a token written into a repaired block (exact_slot >= 0)
// also stores its exact key (bf16, 8 channels per lane) in the block's pool
// row, and its witness is 0 (the decode takes c = 0 there).  The host refuses
// float32 keys for a cache with exact_slot set, so only the bf16 instance
// copies.  es: the block's exact_slot entry (null: no pool).  Returns whether
// the row's block is repaired.
template <typename T>
__device__ __forceinline__ bool repaired_row(const wc_cache& c, const int32_t* es, int64_t off, const T* krow,
                                             int lane16) {
  if (!es) return false;
  const int32_t s = *es;
  if (s < 0) return false;
  if constexpr (sizeof(T) == 2) {
    const uint4 x = *reinterpret_cast<const uint4*>(krow);
    *reinterpret_cast<uint4*>(c.exact_pool + ((int64_t)s * 16 + off) * 128 + 8 * lane16) = x;
  }
  return true;
}

// Element base + e of p.  W32: the launch's every in-layer offset e (in
// bytes) fits in 32 bits, which the host checks; then each access takes the
// wave-uniform p + base and one 32-bit lane offset, not a 64-bit address
// computed per lane.
template <bool W32, typename P>
__device__ __forceinline__ P* at(P* p, int64_t base, typename std::conditional<W32, uint32_t, int64_t>::type e) {
  if (!W32) return p + base + e;
  using B = typename std::conditional<std::is_const<P>::value, const char, char>::type;
  return reinterpret_cast<P*>(reinterpret_cast<B*>(p + base) + (uint32_t)(e * (uint32_t)sizeof(P)));
}

// Grid (ceil(n_tok / 16), Hkv, n_layers): 16 consecutive tokens of one KV
// head per workgroup (no index division).  When the workgroup's 16 rows are
// the 16 tokens of one page in order (a prefill written through this call),
// the page's code blocks are assembled in LDS and leave as whole 16-byte
// lines, as in the page path; otherwise each row stores its own bytes (a
// token's value codes are every fourth byte of its block).
template <typename T, int SCHEME, bool OUTL, bool W32>
__global__ void __launch_bounds__(256) write_rows_kernel(wc_cache c, const T* __restrict__ kin,
                                                         const T* __restrict__ vin, RowArgs a) {
  __shared__ __align__(16) uint8_t sK[2048];
  __shared__ __align__(16) uint8_t sV[2048];
  using IX = typename std::conditional<W32, uint32_t, int64_t>::type;   // in-layer offsets
  const int lane16 = threadIdx.x & 15, j = threadIdx.x >> 4;
  const int64_t tok0 = (int64_t)blockIdx.x * 16;                      // < n_tok
  const int64_t tok = tok0 + j;
  const bool live = tok < a.n_tok;
  const IX i = live ? (IX)tok : (IX)0;        // (n_tok <= 2^26)
  const int g = blockIdx.y, l = blockIdx.z;
  const int layer = a.layer0 + l;
  const int64_t slot = *at<W32>(a.slot, 0, i);
  const IX page = (IX)(slot / 16), off = (IX)(slot % 16);
  const int32_t p = *at<W32>(a.pos, 0, i);
  const IX in_e = (i * (IX)a.hkv + (IX)g) * 128 + (IX)(8 * lane16);
  const int64_t in_base = (int64_t)l * a.layer_stride;
  const T* krow = at<W32>(kin, in_base, in_e);
  const T* vrow = at<W32>(vin, in_base, in_e);
  // the input rows and the first row's slot are requested before anything
  // waits on the index loads above
  const Raw8<T> rk = load_raw8<T>(krow), rv = load_raw8<T>(vrow);
  const int64_t s0 = *at<W32>(a.slot, 0, (IX)tok0);
  const int64_t lpg = (int64_t)layer * a.num_pages * a.hkv;         // the layer's first page-head block
  const IX pgl = page * (IX)a.hkv + (IX)g;                           // the row's block within the layer

  uint32_t omask = 0;
  int ochan = -1;
  if (OUTL) bypass_lanes(c, layer, a.hkv, g, lane16, omask, ochan);
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  if (SCHEME == WC_DITHER_INT8) {
    // the wave's four rows usually belong to one sequence: then its key is
    // chained once, in scalar registers
    const uint64_t sd = *at<W32>(a.seed, 0, i);
    const uint32_t lo = (uint32_t)sd, hi = (uint32_t)(sd >> 32);
    const uint32_t lo0 = __builtin_amdgcn_readfirstlane(lo), hi0 = __builtin_amdgcn_readfirstlane(hi);
    uint32_t key;
    if (__builtin_amdgcn_ballot_w64(lo != lo0 || hi != hi0) == 0)
      key = stream_key(((uint64_t)hi0 << 32) | lo0, (uint32_t)layer, (uint32_t)g);
    else
      key = stream_key(sd, (uint32_t)layer, (uint32_t)g);
#pragma unroll
    for (int w = 0; w < 4; ++w) words[w] = pcg_out_sdwa((key + (uint32_t)(64 * p + 4 * lane16 + w)) * kPcgMul + kPcgInc);
  }
  const RowQ o = quant_row<T, SCHEME>(rk, rv, words, omask);
  // whole page: row j is token j of the page that holds the first row's slot
  const bool whole = __syncthreads_and(live && slot == s0 + j && (s0 & 15) == 0);   // workgroup-uniform
  constexpr bool SC = SCHEME == WC_DITHER_INT8 || SCHEME == WC_RTN_INT8;
  // keys: channels 8 lane16 .. +7 of token off: half (lane16 % 4) / 2, 32-channel
  // group lane16 / 4, bytes 8 (lane16 % 2) .. of the token's 16-byte chunk;
  // values: channel c = 8 lane16 + k of token off goes to half (c % 32) / 16,
  // token group off / 4, lane row 4 (c / 32) + c % 4, word (c % 16) / 4, byte
  // off % 4 (the decode's value tiles)
  const int kin_blk = ((lane16 & 3) >> 1) * 1024 + (lane16 >> 2) * 256 + 8 * (lane16 & 1);
  const int vin_blk = ((lane16 >> 1) & 1) * 1024 + (lane16 >> 2) * 64 + (lane16 & 1) * 8;
  if (whole) {
    *reinterpret_cast<uint2*>(sK + kin_blk + j * 16) = make_uint2(o.kp[0], o.kp[1]);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      sV[vin_blk + (j >> 2) * 256 + (k & 3) * 16 + (k >> 2) * 4 + (j & 3)] = (uint8_t)(o.vp[k >> 2] >> (8 * (k & 3)));
  } else if (live) {
    uint8_t* kc = at<W32>(reinterpret_cast<uint8_t*>(c.k_codes), lpg * 2048, pgl * 2048 + (IX)kin_blk + off * 16);
    *reinterpret_cast<uint2*>(kc) = make_uint2(o.kp[0], o.kp[1]);
    uint8_t* vc = at<W32>(reinterpret_cast<uint8_t*>(c.v_codes), lpg * 2048,
                          pgl * 2048 + (IX)vin_blk + (off >> 2) * 256 + (off & 3));
#pragma unroll
    for (int k = 0; k < 8; ++k) vc[(k & 3) * 16 + (k >> 2) * 4] = (uint8_t)(o.vp[k >> 2] >> (8 * (k & 3)));
  }
  if (live) {
    const int32_t* es = c.exact_slot ? at<W32>((const int32_t*)c.exact_slot, lpg, pgl) : nullptr;
    const bool rep = repaired_row<T>(c, es, (int64_t)off, krow, lane16);
    const IX row = pgl * 16 + off;                                   // (block, token) within the layer
    if (lane16 < 8) *at<W32>(c.witness, lpg * 128, row * 8 + (IX)lane16) = rep ? 0.0f : o.w;
    if (SC && lane16 == 0) {
      *at<W32>(c.k_scale, lpg * 16, row) = o.ks;
      *at<W32>(c.v_scale, lpg * 16, row) = o.vs;
    }
    if (c.v_witness && lane16 == 0) *at<W32>(c.v_witness, lpg * 16, row) = o.wv;
    if (OUTL && ochan >= 0)
      *at<W32>(c.k_outlier, lpg * 16 * c.num_outliers, row * (IX)c.num_outliers + (IX)lane16) =
          reinterpret_cast<const uint16_t*>(krow - 8 * lane16)[ochan];
  }
  if (whole) {
    __syncthreads();
    // threads 0..127 the key block, 128..255 the value block, 16 bytes each
    const int t = threadIdx.x & 127;
    const IX pg0 = (IX)(s0 / 16) * (IX)a.hkv + (IX)g;
    uint8_t* dst = at<W32>(reinterpret_cast<uint8_t*>(threadIdx.x < 128 ? c.k_codes : c.v_codes), lpg * 2048,
                           pg0 * 2048 + (IX)(16 * t));
    __builtin_nontemporal_store(*reinterpret_cast<const nt_u4*>((threadIdx.x < 128 ? sK : sV) + 16 * t),
                                reinterpret_cast<nt_u4*>(dst));
  }
}

// Whole pages (prefill): one workgroup per (layer, page, KV head) block, row
// = token j of the page.  The same arithmetic as write_rows_kernel; the code
// blocks are assembled in LDS and leave as 2 KB of 16-byte stores each.
struct PageArgs {
  int64_t n_pages;
  int64_t layer_stride;
  int64_t num_pages;
  int hkv;
  int layer0;
  const int32_t* pages;
  const int32_t* pos0;
  const uint64_t* seed;
};

template <typename T, int SCHEME, bool OUTL>
__global__ void __launch_bounds__(256) write_pages_kernel(wc_cache c, const T* __restrict__ kin,
                                                          const T* __restrict__ vin, PageArgs a) {
  __shared__ __align__(16) uint8_t sK[2048];
  __shared__ __align__(16) uint8_t sV[2048];
  const int lane16 = threadIdx.x & 15, j = threadIdx.x >> 4;
  const int64_t pi = blockIdx.x;                  // grid (n_pages, Hkv, n_layers)
  const int g = blockIdx.y, l = blockIdx.z;
  const int layer = a.layer0 + l;
  const int64_t i = pi * 16 + j;                  // input token
  const int32_t p = a.pos0[pi] + j;
  const int64_t in_off = (int64_t)l * a.layer_stride + (i * a.hkv + g) * 128 + 8 * lane16;
  const int64_t pg = ((int64_t)layer * a.num_pages + a.pages[pi]) * a.hkv + g;

  uint32_t omask = 0;
  int ochan = -1;
  if (OUTL) bypass_lanes(c, layer, a.hkv, g, lane16, omask, ochan);
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  if (SCHEME == WC_DITHER_INT8) {
    const uint32_t key = stream_key(a.seed[pi], (uint32_t)layer, (uint32_t)g);
#pragma unroll
    for (int w = 0; w < 4; ++w) words[w] = pcg_out_sdwa((key + (uint32_t)(64 * p + 4 * lane16 + w)) * kPcgMul + kPcgInc);
  }
  const RowQ o = quant_row<T, SCHEME>(load_raw8<T>(kin + in_off), load_raw8<T>(vin + in_off), words, omask);
  constexpr bool SC = SCHEME == WC_DITHER_INT8 || SCHEME == WC_RTN_INT8;
  *reinterpret_cast<uint2*>(sK + ((lane16 & 3) >> 1) * 1024 + (lane16 >> 2) * 256 + j * 16 + 8 * (lane16 & 1)) =
      make_uint2(o.kp[0], o.kp[1]);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    sV[((lane16 >> 1) & 1) * 1024 + (j >> 2) * 256 + (lane16 >> 2) * 64 + (k & 3) * 16 + (lane16 & 1) * 8 +
       (k >> 2) * 4 + (j & 3)] = (uint8_t)(o.vp[k >> 2] >> (8 * (k & 3)));
  const bool rep = repaired_row<T>(c, c.exact_slot ? c.exact_slot + pg : nullptr, j, kin + in_off, lane16);
  if (lane16 < 8) c.witness[(pg * 16 + j) * 8 + lane16] = rep ? 0.0f : o.w;
  if (SC && lane16 == 0) {
    c.k_scale[pg * 16 + j] = o.ks;
    c.v_scale[pg * 16 + j] = o.vs;
  }
  if (c.v_witness && lane16 == 0) c.v_witness[pg * 16 + j] = o.wv;
  if (OUTL && ochan >= 0)
    c.k_outlier[(pg * 16 + j) * c.num_outliers + lane16] = reinterpret_cast<const uint16_t*>(kin)[in_off - 8 * lane16 + ochan];
  __syncthreads();
  const int t = threadIdx.x & 127;
  uint8_t* dst = reinterpret_cast<uint8_t*>(threadIdx.x < 128 ? c.k_codes : c.v_codes) + pg * 2048 + 16 * t;
  __builtin_nontemporal_store(*reinterpret_cast<const nt_u4*>((threadIdx.x < 128 ? sK : sV) + 16 * t),
                              reinterpret_cast<nt_u4*>(dst));
}

// 16-bit store: the scheme's outputs (bf16) copied into the decode layouts,
// witness 0 (wc_witness writes the scheme's own).  16 lanes per row, 8
// channels each, as above.
__global__ void __launch_bounds__(256) write_bf16_kernel(wc_cache c, const uint16_t* __restrict__ kin,
                                                         const uint16_t* __restrict__ vin, RowArgs a) {
  const int lane16 = threadIdx.x & 15;
  const int64_t i = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);     // grid as write_rows_kernel
  if (i >= a.n_tok) return;
  const int g = blockIdx.y, l = blockIdx.z;
  const int64_t slot = a.slot[i];
  const int64_t page = slot / 16, off = slot % 16;
  const int64_t in_off = (int64_t)l * a.layer_stride + (i * a.hkv + g) * 128 + 8 * lane16;
  const int64_t pg = ((int64_t)(a.layer0 + l) * a.num_pages + page) * a.hkv + g;
  const uint4 kv = *reinterpret_cast<const uint4*>(kin + in_off);
  const uint4 vv = *reinterpret_cast<const uint4*>(vin + in_off);
  // keys: channels 8 lane16 .. +7 of token off at [(c%32)/8][c/32][off][c%8]
  uint8_t* kb = reinterpret_cast<uint8_t*>(c.k_codes) + pg * 4096;
  *reinterpret_cast<uint4*>(kb + (lane16 & 3) * 1024 + (lane16 >> 2) * 256 + off * 16) = kv;
  // values: channel 8 lane16 + e at [e/2][off/4][lane16][e%2][off%4]
  uint16_t* vb = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(c.v_codes) + pg * 4096);
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    vb[(e >> 1) * 512 + (off >> 2) * 128 + lane16 * 8 + (e & 1) * 4 + (off & 3)] =
        (uint16_t)((e & 1) ? w[e >> 1] >> 16 : w[e >> 1] & 0xFFFFu);
  if (lane16 < 8) c.witness[(pg * 16 + off) * 8 + lane16] = 0.0f;
  if (c.v_witness && lane16 == 0) c.v_witness[pg * 16 + off] = 0.0f;
}

// Witness of an arbitrary scheme's output: keys w_{t,b} = ||xhat - x|| over
// band b; values (VAL) ||xhat - x|| over the whole row.
template <typename T, bool VAL>
__global__ void __launch_bounds__(256) witness_kernel(wc_cache c, const T* __restrict__ x, const T* __restrict__ xh,
                                                      RowArgs a) {
  const int lane16 = threadIdx.x & 15;
  const int64_t tok = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);   // grid as write_rows_kernel
  const bool live = tok < a.n_tok;
  const int64_t i = live ? tok : 0;
  const int g = blockIdx.y, l = blockIdx.z;
  const int64_t in_off = (int64_t)l * a.layer_stride + (i * a.hkv + g) * 128 + 8 * lane16;
  float xv[8], hv[8];
  load8<T>(x + in_off, xv);
  load8<T>(xh + in_off, hv);
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float r = hv[k] - xv[k];
    ss = fmaf(r, r, ss);
  }
  if (VAL) {
    ss = row16_sum(ss);
    if (live && lane16 == 0) {
      const int64_t slot = a.slot[i];
      const int64_t pg = ((int64_t)(a.layer0 + l) * a.num_pages + slot / 16) * a.hkv + g;
      c.v_witness[pg * 16 + slot % 16] = sqrtf(ss) * kWitnessGuard;
    }
    return;
  }
  const float tot = ss + dpp_f<kRowRor8>(ss);
  if (!live) return;
  const int64_t slot = a.slot[i];
  const int64_t pg = ((int64_t)(a.layer0 + l) * a.num_pages + slot / 16) * a.hkv + g;
  // a repaired block: the exact key x to the pool row, witness 0
  const bool rep = repaired_row<T>(c, c.exact_slot ? c.exact_slot + pg : nullptr, slot % 16, x + in_off, lane16);
  if (lane16 < 8) c.witness[(pg * 16 + slot % 16) * 8 + lane16] = rep ? 0.0f : sqrtf(tot) * kWitnessGuard;
}

// ---------------------------------------------------------------- 2-bit (KIVI-style)
// One workgroup per (layer, 32-token page, KV head).  Keys are grouped over
// the 32 tokens of each channel, values over 32 channels of each token.
template <typename T>
__device__ __forceinline__ float ldf(const T* p);
template <>
__device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ void quant2(float x, float mn, float scale, float inv, uint32_t& code, float& xhat) {
  float q = 0.0f;
  if (scale != 0.0f) q = fminf(fmaxf(rintf(mul_rn(x - mn, inv)), 0.0f), 3.0f);
  code = (uint32_t)q;
  xhat = add_rn(mn, mul_rn(q, scale));
}

template <typename T>
__global__ void __launch_bounds__(256) write_kivi2_kernel(wc_cache c, const T* __restrict__ kin,
                                                          const T* __restrict__ vin, RowArgs a) {
  __shared__ float xs[32][129];
  __shared__ float red[2][2][128];
  const int t = threadIdx.x;
  const int64_t grp = blockIdx.x;                // grid (n_tok / 32, Hkv, n_layers)
  const int g = blockIdx.y, l = blockIdx.z;
  const int layer = a.layer0 + l;
  const int64_t i0 = grp * 32;
  const int64_t page = a.slot[i0] / 32;
  const int64_t pg = ((int64_t)layer * a.num_pages + page) * a.hkv + g;
  const T* kb = kin + (int64_t)l * a.layer_stride;
  const T* vb = vin + (int64_t)l * a.layer_stride;

  // every load of the workgroup first: this thread's 16 value channels (token
  // t / 8, channels 16 (t % 8) ..) and its two pieces of the 32 x 128 key tile
  // (8 channels per 16-byte load), so that the value rows' latency passes
  // while the keys are processed
  const int vtok = t >> 3, vpart = t & 7;
  const T* vsrc = vb + ((i0 + vtok) * a.hkv + g) * 128 + 16 * vpart;
  const Raw8<T> rv0 = load_raw8<T>(vsrc), rv1 = load_raw8<T>(vsrc + 8);
  Raw8<T> rk[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = t + 256 * u, tok = e >> 4, c8 = (e & 15) * 8;
    rk[u] = load_raw8<T>(kb + ((i0 + tok) * a.hkv + g) * 128 + c8);
  }
  // keys: stage the tile, per-channel min/max over the 32 tokens
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = t + 256 * u, tok = e >> 4, c8 = (e & 15) * 8;
    float x8[8];
    unpack8(rk[u], x8);
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[tok][c8 + j] = x8[j];
  }
  __syncthreads();
  const int ch = t & 127, h = t >> 7;
  float mn = xs[16 * h][ch], mx = mn;
  for (int k = 1; k < 16; ++k) {
    mn = fminf(mn, xs[16 * h + k][ch]);
    mx = fmaxf(mx, xs[16 * h + k][ch]);
  }
  red[0][h][ch] = mn;
  red[1][h][ch] = mx;
  __syncthreads();
  mn = fminf(red[0][0][ch], red[0][1][ch]);
  mx = fmaxf(red[1][0][ch], red[1][1][ch]);
  const float scale = div_rn(mx - mn, 3.0f);
  const float inv = scale != 0.0f ? div_rn(1.0f, scale) : 0.0f;
  uint32_t packed = 0;
  float res[16];
  for (int k = 0; k < 16; ++k) {
    uint32_t code;
    float xh;
    float x = xs[16 * h + k][ch];
    quant2(x, mn, scale, inv, code, xh);
    packed |= code << (2 * k);
    res[k] = xh - x;
  }
  uint8_t* kc = reinterpret_cast<uint8_t*>(c.k_codes) + pg * 1024 + ch * 8 + 4 * h;
  *reinterpret_cast<uint32_t*>(kc) = packed;
  if (h == 0) {
    c.k_aux[(pg * 128 + ch) * 2 + 0] = scale;
    c.k_aux[(pg * 128 + ch) * 2 + 1] = mn;
  }
  __syncthreads();
  for (int k = 0; k < 16; ++k) xs[16 * h + k][ch] = res[k];
  __syncthreads();
  {
    const int tok = t >> 3, b = t & 7;
    float ss = 0.0f;
    for (int k = 0; k < 8; ++k) {
      float r0 = xs[tok][8 * b + k];
      ss = fmaf(r0, r0, ss);
    }
    float s2 = 0.0f;
    for (int k = 0; k < 8; ++k) {
      float r1 = xs[tok][64 + 8 * b + k];
      s2 = fmaf(r1, r1, s2);
    }
    c.witness[(pg * 32 + tok) * 8 + b] = sqrtf(ss + s2) * kWitnessGuard;
  }
  // values: groups of 32 channels of one token; thread = (token, 16-channel half-group)
  {
    const int tok = vtok, part = vpart;
    float x[16];
    unpack8(rv0, *reinterpret_cast<float(*)[8]>(&x[0]));
    unpack8(rv1, *reinterpret_cast<float(*)[8]>(&x[8]));
    float vmn = x[0], vmx = x[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) {
      vmn = fminf(vmn, x[k]);
      vmx = fmaxf(vmx, x[k]);
    }
    vmn = fminf(vmn, __shfl_xor(vmn, 1, 64));
    vmx = fmaxf(vmx, __shfl_xor(vmx, 1, 64));
    const float vs = div_rn(vmx - vmn, 3.0f);
    const float vinv = vs != 0.0f ? div_rn(1.0f, vs) : 0.0f;
    uint32_t pk = 0;
    float vss = 0.0f;
    for (int k = 0; k < 16; ++k) {
      uint32_t code;
      float xh;
      quant2(x[k], vmn, vs, vinv, code, xh);
      pk |= code << (2 * k);
      const float rv = xh - x[k];
      vss = fmaf(rv, rv, vss);
    }
    // value witness of the token: its 8 threads (t & 7) hold 16 channels each
    vss += __shfl_xor(vss, 1, 64);
    vss += __shfl_xor(vss, 2, 64);
    vss += __shfl_xor(vss, 4, 64);
    if (c.v_witness && part == 0) c.v_witness[pg * 32 + tok] = sqrtf(vss) * kWitnessGuard;
    uint8_t* vc = reinterpret_cast<uint8_t*>(c.v_codes) + pg * 1024 + tok * 32 + 4 * part;
    *reinterpret_cast<uint32_t*>(vc) = pk;
    if ((part & 1) == 0) {
      c.v_aux[((pg * 32 + tok) * 4 + part / 2) * 2 + 0] = vs;
      c.v_aux[((pg * 32 + tok) * 4 + part / 2) * 2 + 1] = vmn;
    }
  }
}

// ---------------------------------------------------------------- outlier channels
// One workgroup of 128 threads per (KV head, layer): thread c accumulates
// E_c = sum_t x_{t,c}^2 in float32 in token order (loads eight tokens ahead),
// then ranks the channels by (E desc, c asc) through LDS; the m first are
// written in ascending channel order.
template <typename T>
__global__ void __launch_bounds__(128) outlier_select_kernel(const T* __restrict__ x, int64_t n_tok, int hkv,
                                                             int64_t layer_stride, int m, int32_t* out) {
  __shared__ float e[128];
  __shared__ int sel[128];
  const int c = threadIdx.x, g = blockIdx.x, l = blockIdx.y;
  const T* p = x + (int64_t)l * layer_stride + (int64_t)g * 128 + c;
  const int64_t stride = (int64_t)hkv * 128;
  float acc = 0.0f;
  int64_t t = 0;
  for (; t + 8 <= n_tok; t += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ldf<T>(p + (t + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = add_rn(acc, mul_rn(v[u], v[u]));
  }
  for (; t < n_tok; ++t) {
    const float v = ldf<T>(p + t * stride);
    acc = add_rn(acc, mul_rn(v, v));
  }
  if (acc != acc) acc = INFINITY;              // NaN ranks as +inf: the order stays total
  e[c] = acc;
  __syncthreads();
  int rank = 0;
  for (int o = 0; o < 128; ++o) {
    const float eo = e[o];
    rank += (eo > acc || (eo == acc && o < c)) ? 1 : 0;
  }
  sel[c] = rank < m ? 1 : 0;
  __syncthreads();
  if (rank < m) {
    int at = 0;
    for (int o = 0; o < c; ++o) at += sel[o];
    if (at < m) out[((int64_t)l * hkv + g) * m + at] = c;
  }
}

// ---------------------------------------------------------------- dither fill (test hook)
__global__ void dither_fill_kernel(uint32_t key, int64_t pos0, int64_t n_pos, uint16_t* out) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_pos * 128) return;
  const int64_t t = pos0 + e / 128;
  const int c = (int)(e % 128);
  const uint32_t word = pcg(key + (uint32_t)(64 * t + (c >> 1)));
  out[e] = (uint16_t)((c & 1) ? word >> 16 : word & 0xFFFFu);
}

}  // namespace wc

using namespace wc;

extern "C" int wc_write_kv(const wc_cache* cache, int layer0, int n_layers, const void* k, const void* v,
                           int in_dtype, int64_t n_tok, int64_t layer_stride, const int64_t* slot,
                           const int32_t* pos, const uint64_t* seed, void* stream) {
  if (!cache || (n_tok != 0 && (!k || !v || !slot || !pos || !seed))) {
    set_error("wc_write_kv: null pointer");
    return WC_EINVAL;
  }
  const wc_cache& c = *cache;
  if (c.head_dim != 128 || c.num_bands != 8 || c.num_kv_heads < 1 || c.num_layers < 1 || c.num_pages < 1) {
    set_error("wc_write_kv: need head_dim 128, 8 bands, >= 1 KV head, layer and page");
    return WC_EUNSUPPORTED;
  }
  if (layer0 < 0 || n_layers < 1 || n_layers > 65535 || layer0 + n_layers > c.num_layers || n_tok < 0 ||
      c.num_kv_heads > 65535) {
    set_error("wc_write_kv: layer range, head count or token count out of range");
    return WC_EINVAL;
  }
  if (in_dtype != WC_F32 && in_dtype != WC_BF16) {
    set_error("wc_write_kv: in_dtype must be WC_F32 or WC_BF16");
    return WC_EUNSUPPORTED;
  }
  if (n_layers > 1 && layer_stride < n_tok * c.num_kv_heads * 128) {
    set_error("wc_write_kv: layer_stride smaller than one layer");
    return WC_EINVAL;
  }
  if (!c.k_codes || !c.v_codes || !c.witness) {
    set_error("wc_write_kv: cache codes and witness must be set");
    return WC_EINVAL;
  }
  if (n_tok > (int64_t(1) << 26)) {
    set_error("wc_write_kv: at most 2^26 tokens per call");
    return WC_EINVAL;
  }
  if (c.exact_slot && in_dtype == WC_F32) {
    set_error("wc_write_kv: a cache with an exact pool (exact_slot set) takes bf16 keys: the exact store is bf16");
    return WC_EUNSUPPORTED;
  }
  if (c.exact_slot && !c.exact_pool) {
    set_error("wc_write_kv: exact_slot set without exact_pool");
    return WC_EINVAL;
  }
  RowArgs a{n_tok, layer_stride, c.num_pages, c.num_kv_heads, layer0, n_layers, slot, pos, seed};
  hipStream_t st = (hipStream_t)stream;
  if (n_tok == 0) return WC_OK;
  if (c.scheme == WC_BF16_STORE) {
    if (c.page_size != 16 || in_dtype != WC_BF16 || c.num_outliers != 0) {
      set_error("wc_write_kv: the 16-bit store takes bf16 input and 16-token pages, no outlier bypass");
      return WC_EUNSUPPORTED;
    }
    hipLaunchKernelGGL(write_bf16_kernel, dim3((unsigned)((n_tok + 15) / 16), (unsigned)c.num_kv_heads,
                       (unsigned)n_layers), dim3(256), 0, st, c, (const uint16_t*)k, (const uint16_t*)v, a);
    return check_launch("wc_write_kv");
  }
  if (c.scheme == WC_DITHER_INT8 || c.scheme == WC_FP8_E4M3 || c.scheme == WC_RTN_INT8) {
    if (c.page_size != 16) {
      set_error("wc_write_kv: INT8 and fp8 caches use 16-token pages");
      return WC_EUNSUPPORTED;
    }
    if ((c.scheme == WC_DITHER_INT8 || c.scheme == WC_RTN_INT8) && (!c.k_scale || !c.v_scale)) {
      set_error("wc_write_kv: INT8 cache needs k_scale and v_scale");
      return WC_EINVAL;
    }
    if (c.num_outliers != 0) {
      if (c.scheme != WC_DITHER_INT8 || (c.num_outliers != 8 && c.num_outliers != 16)) {
        set_error("wc_write_kv: the outlier bypass needs the dithered INT8 scheme and m = 8 or 16");
        return WC_EUNSUPPORTED;
      }
      if (in_dtype != WC_BF16) {
        set_error("wc_write_kv: the outlier bypass stores bf16 keys: input must be WC_BF16");
        return WC_EUNSUPPORTED;
      }
      if (!c.outlier_ch || !c.k_outlier) {
        set_error("wc_write_kv: outlier bypass needs outlier_ch and k_outlier");
        return WC_EINVAL;
      }
    }
    dim3 grid((unsigned)((n_tok + 15) / 16), (unsigned)c.num_kv_heads, (unsigned)n_layers);
    // 32-bit in-layer offsets when one layer's code array and one layer of
    // input fit in 4 GB (the index arrays do: n_tok <= 2^26)
    const int64_t esize = in_dtype == WC_BF16 ? 2 : 4;
    const bool w32 = c.num_pages * c.num_kv_heads * 2048 <= (int64_t(1) << 32) &&
                     n_tok * c.num_kv_heads * 128 * esize <= (int64_t(1) << 32);
#define WC_ROWS(T, SCH, OU)                                                                                    \
  do {                                                                                                         \
    if (w32)                                                                                                   \
      hipLaunchKernelGGL((write_rows_kernel<T, SCH, OU, true>), grid, dim3(256), 0, st, c, (const T*)k,      \
                         (const T*)v, a);                                                                      \
    else                                                                                                       \
      hipLaunchKernelGGL((write_rows_kernel<T, SCH, OU, false>), grid, dim3(256), 0, st, c, (const T*)k,     \
                         (const T*)v, a);                                                                      \
  } while (0)
    const bool bf = in_dtype == WC_BF16;
    if (c.scheme == WC_DITHER_INT8) {
      if (c.num_outliers != 0) WC_ROWS(uint16_t, WC_DITHER_INT8, true);
      else if (bf) WC_ROWS(uint16_t, WC_DITHER_INT8, false);
      else WC_ROWS(float, WC_DITHER_INT8, false);
    } else if (c.scheme == WC_RTN_INT8) {
      if (bf) WC_ROWS(uint16_t, WC_RTN_INT8, false); else WC_ROWS(float, WC_RTN_INT8, false);
    } else {
      if (bf) WC_ROWS(uint16_t, WC_FP8_E4M3, false); else WC_ROWS(float, WC_FP8_E4M3, false);
    }
#undef WC_ROWS
    return check_launch("wc_write_kv");
  }
  if (c.scheme == WC_KIVI2) {
    if (c.page_size != 32 || (n_tok % 32) != 0) {
      set_error("wc_write_kv: 2-bit cache needs 32-token pages and whole pages of tokens");
      return WC_EUNSUPPORTED;
    }
    if (!c.k_aux || !c.v_aux) {
      set_error("wc_write_kv: 2-bit cache needs k_aux and v_aux");
      return WC_EINVAL;
    }
    dim3 grid((unsigned)(n_tok / 32), (unsigned)c.num_kv_heads, (unsigned)n_layers);
    if (in_dtype == WC_BF16)
      hipLaunchKernelGGL((write_kivi2_kernel<uint16_t>), grid, dim3(256), 0, st, c, (const uint16_t*)k,
                         (const uint16_t*)v, a);
    else
      hipLaunchKernelGGL((write_kivi2_kernel<float>), grid, dim3(256), 0, st, c, (const float*)k,
                         (const float*)v, a);
    return check_launch("wc_write_kv");
  }
  set_error("wc_write_kv: unknown scheme %d", c.scheme);
  return WC_EUNSUPPORTED;
}

extern "C" int wc_write_kv_pages(const wc_cache* cache, int layer0, int n_layers, const void* k, const void* v,
                                 int in_dtype, int64_t n_pages, int64_t layer_stride, const int32_t* pages,
                                 const int32_t* pos0, const uint64_t* seed, void* stream) {
  if (!cache || (n_pages != 0 && (!k || !v || !pages || !pos0 || !seed))) {
    set_error("wc_write_kv_pages: null pointer");
    return WC_EINVAL;
  }
  const wc_cache& c = *cache;
  if (c.head_dim != 128 || c.num_bands != 8 || c.num_kv_heads < 1 || c.num_layers < 1 || c.num_pages < 1 ||
      c.page_size != 16) {
    set_error("wc_write_kv_pages: need head_dim 128, 8 bands, 16-token pages");
    return WC_EUNSUPPORTED;
  }
  if (c.scheme != WC_DITHER_INT8 && c.scheme != WC_FP8_E4M3 && c.scheme != WC_RTN_INT8) {
    set_error("wc_write_kv_pages: scheme %d writes through wc_write_kv", c.scheme);
    return WC_EUNSUPPORTED;
  }
  if (layer0 < 0 || n_layers < 1 || n_layers > 65535 || layer0 + n_layers > c.num_layers || n_pages < 0 ||
      n_pages * 16 > (int64_t(1) << 26) || c.num_kv_heads > 65535) {
    set_error("wc_write_kv_pages: layer range or page count out of range");
    return WC_EINVAL;
  }
  if (in_dtype != WC_F32 && in_dtype != WC_BF16) {
    set_error("wc_write_kv_pages: in_dtype must be WC_F32 or WC_BF16");
    return WC_EUNSUPPORTED;
  }
  if (n_layers > 1 && layer_stride < n_pages * 16 * c.num_kv_heads * 128) {
    set_error("wc_write_kv_pages: layer_stride smaller than one layer");
    return WC_EINVAL;
  }
  if (!c.k_codes || !c.v_codes || !c.witness ||
      ((c.scheme == WC_DITHER_INT8 || c.scheme == WC_RTN_INT8) && (!c.k_scale || !c.v_scale))) {
    set_error("wc_write_kv_pages: cache codes, scales and witness must be set");
    return WC_EINVAL;
  }
  if (c.exact_slot && in_dtype == WC_F32) {
    set_error("wc_write_kv_pages: a cache with an exact pool (exact_slot set) takes bf16 keys: the exact store is bf16");
    return WC_EUNSUPPORTED;
  }
  if (c.exact_slot && !c.exact_pool) {
    set_error("wc_write_kv_pages: exact_slot set without exact_pool");
    return WC_EINVAL;
  }
  if (c.num_outliers != 0) {
    if (c.scheme != WC_DITHER_INT8 || (c.num_outliers != 8 && c.num_outliers != 16)) {
      set_error("wc_write_kv_pages: the outlier bypass needs the dithered INT8 scheme and m = 8 or 16");
      return WC_EUNSUPPORTED;
    }
    if (in_dtype != WC_BF16) {
      set_error("wc_write_kv_pages: the outlier bypass stores bf16 keys: input must be WC_BF16");
      return WC_EUNSUPPORTED;
    }
    if (!c.outlier_ch || !c.k_outlier) {
      set_error("wc_write_kv_pages: outlier bypass needs outlier_ch and k_outlier");
      return WC_EINVAL;
    }
  }
  if (n_pages == 0) return WC_OK;
  PageArgs a{n_pages, layer_stride, c.num_pages, c.num_kv_heads, layer0, pages, pos0, seed};
  dim3 grid((unsigned)n_pages, (unsigned)c.num_kv_heads, (unsigned)n_layers);
  hipStream_t st = (hipStream_t)stream;
  const bool bf = in_dtype == WC_BF16;
#define WC_PAGES(T, SCH, OU) hipLaunchKernelGGL((write_pages_kernel<T, SCH, OU>), grid, dim3(256), 0, st, c, \
                                                (const T*)k, (const T*)v, a)
  if (c.scheme == WC_DITHER_INT8) {
    if (c.num_outliers != 0) WC_PAGES(uint16_t, WC_DITHER_INT8, true);
    else if (bf) WC_PAGES(uint16_t, WC_DITHER_INT8, false);
    else WC_PAGES(float, WC_DITHER_INT8, false);
  } else if (c.scheme == WC_RTN_INT8) {
    if (bf) WC_PAGES(uint16_t, WC_RTN_INT8, false); else WC_PAGES(float, WC_RTN_INT8, false);
  } else {
    if (bf) WC_PAGES(uint16_t, WC_FP8_E4M3, false); else WC_PAGES(float, WC_FP8_E4M3, false);
  }
#undef WC_PAGES
  return check_launch("wc_write_kv_pages");
}

extern "C" int wc_witness(const wc_cache* cache, int layer0, int n_layers, const void* x, const void* xhat,
                          int in_dtype, int64_t n_tok, int64_t layer_stride, const int64_t* slot, int values,
                          void* stream) {
  if (!cache || (n_tok != 0 && (!x || !xhat || !slot))) {
    set_error("wc_witness: null pointer");
    return WC_EINVAL;
  }
  const wc_cache& c = *cache;
  if (c.head_dim != 128 || c.num_bands != 8 || c.page_size != 16 || c.num_kv_heads < 1 || c.num_pages < 1) {
    set_error("wc_witness: need head_dim 128, 8 bands, 16-token pages");
    return WC_EUNSUPPORTED;
  }
  if (values != 0 && values != 1) {
    set_error("wc_witness: values must be 0 (keys) or 1 (values)");
    return WC_EINVAL;
  }
  if (values ? !c.v_witness : !c.witness) {
    set_error("wc_witness: cache %s witness not set", values ? "value" : "key");
    return WC_EINVAL;
  }
  if (layer0 < 0 || n_layers < 1 || n_layers > 65535 || c.num_kv_heads > 65535 ||
      layer0 + n_layers > c.num_layers || n_tok < 0 || n_tok > (int64_t(1) << 30) ||
      (n_layers > 1 && layer_stride < n_tok * c.num_kv_heads * 128)) {
    set_error("wc_witness: layer range, token count or layer stride out of range");
    return WC_EINVAL;
  }
  if (in_dtype != WC_F32 && in_dtype != WC_BF16) {
    set_error("wc_witness: in_dtype must be WC_F32 or WC_BF16");
    return WC_EUNSUPPORTED;
  }
  if (!values && c.exact_slot && in_dtype == WC_F32) {
    set_error("wc_witness: a cache with an exact pool (exact_slot set) takes bf16 keys: the exact store is bf16");
    return WC_EUNSUPPORTED;
  }
  if (!values && c.exact_slot && !c.exact_pool) {
    set_error("wc_witness: exact_slot set without exact_pool");
    return WC_EINVAL;
  }
  if (n_tok == 0) return WC_OK;
  RowArgs a{n_tok, layer_stride, c.num_pages, c.num_kv_heads, layer0, n_layers, slot, nullptr, nullptr};
  dim3 grid((unsigned)((n_tok + 15) / 16), (unsigned)c.num_kv_heads, (unsigned)n_layers);
  hipStream_t st = (hipStream_t)stream;
  if (in_dtype == WC_BF16) {
    if (values)
      hipLaunchKernelGGL((witness_kernel<uint16_t, true>), grid, dim3(256), 0, st, c, (const uint16_t*)x,
                         (const uint16_t*)xhat, a);
    else
      hipLaunchKernelGGL((witness_kernel<uint16_t, false>), grid, dim3(256), 0, st, c, (const uint16_t*)x,
                         (const uint16_t*)xhat, a);
  } else {
    if (values)
      hipLaunchKernelGGL((witness_kernel<float, true>), grid, dim3(256), 0, st, c, (const float*)x,
                         (const float*)xhat, a);
    else
      hipLaunchKernelGGL((witness_kernel<float, false>), grid, dim3(256), 0, st, c, (const float*)x,
                         (const float*)xhat, a);
  }
  return check_launch("wc_witness");
}

extern "C" int wc_outlier_select(const void* x, int in_dtype, int n_layers, int64_t n_tok, int num_kv_heads,
                                 int64_t layer_stride, int m, int32_t* channels, void* stream) {
  if ((!x && n_tok > 0) || !channels) {
    set_error("wc_outlier_select: null pointer");
    return WC_EINVAL;
  }
  if (n_layers < 1 || n_layers > 65535 || n_tok < 0 || num_kv_heads < 1 || m < 1 || m > 128) {
    set_error("wc_outlier_select: need n_layers in 1..65535, n_tok >= 0, num_kv_heads >= 1, m in 1..128");
    return WC_EINVAL;
  }
  if (n_layers > 1 && layer_stride < n_tok * num_kv_heads * 128) {
    set_error("wc_outlier_select: layer_stride smaller than one layer");
    return WC_EINVAL;
  }
  if (in_dtype != WC_F32 && in_dtype != WC_BF16) {
    set_error("wc_outlier_select: in_dtype must be WC_F32 or WC_BF16");
    return WC_EUNSUPPORTED;
  }
  dim3 grid((unsigned)num_kv_heads, (unsigned)n_layers);
  hipStream_t st = (hipStream_t)stream;
  if (in_dtype == WC_BF16)
    hipLaunchKernelGGL((outlier_select_kernel<uint16_t>), grid, dim3(128), 0, st, (const uint16_t*)x, n_tok,
                       num_kv_heads, layer_stride, m, channels);
  else
    hipLaunchKernelGGL((outlier_select_kernel<float>), grid, dim3(128), 0, st, (const float*)x, n_tok,
                       num_kv_heads, layer_stride, m, channels);
  return check_launch("wc_outlier_select");
}

extern "C" int wc_dither_fill(uint64_t seed, int layer, int kv_head, int64_t pos0, int64_t n_pos, uint16_t* out,
                              void* stream) {
  if ((!out && n_pos != 0) || n_pos < 0 || pos0 < 0 || pos0 + n_pos > (int64_t(1) << 26)) {
    set_error("wc_dither_fill: bad arguments");
    return WC_EINVAL;
  }
  if (n_pos == 0) return WC_OK;
  const uint32_t key = stream_key(seed, (uint32_t)layer, (uint32_t)kv_head);
  const int64_t n = n_pos * 128;
  hipLaunchKernelGGL(dither_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, key,
                     pos0, n_pos, out);
  return check_launch("wc_dither_fill");
}

extern "C" const char* wc_last_error(void) { return g_err; }
extern "C" const char* wc_version(void) { return "witcert-mi355x 0.1"; }
