// Fused split-KV decode attention + WitCert meter, and the LSE merge.
//
// WitCert summary: Theorem 2 (Tier A) eps_t <= (1/sqrt d) sum_b ||q_b|| w_{t,b};
// Tier B paragraph: u_t = sqrt(2 varsigma_t^2 log(2S/delta_loc)),
// varsigma_t^2 = (1/d) sum_c q_c^2 s_{c,t}^2 / 12, delta_loc = delta_req/(L H T);
// improvements list: TV <= min(1, (A^2 - 1)/2), A = sum_t p~_t e^{c_t};
// page-in paragraph: the deterministic tanh bound the certificate is compared
// with, taken here as TV <= tanh(max_t c_t / 2) (a logit move of at most c_t
// per token bounds the log-ratio range by 2 max c; the range D gives
// TV <= tanh(D / 4)); the kernel carries max_t c_t per tier;
// implementation paragraph and the paperswithlean Figure 2 caption: output and
// meter in one data pass, LSE-merged across KV splits.
//
// Work decomposition: one workgroup of 4 waves per (sequence b, KV head g,
// split); the waves take the split's 16-token pages round robin and combine
// through LDS at the end.  Inside a wave, lane l is (n = l % 16, k = l / 16):
//
//   QK   S^T[token][head] = Khat[token][:] . Q'[head][:]   (MFMA 16x16x32 f16)
//        A = key codes of token n, channels 32k..32k+31 (one 32 B load);
//        B = the scaled query of head n, same channels.  The dequantized key
//        is s_t (code - xi) with xi = hb 2^-8 + lb 2^-16 - 1/2 (hb, lb the
//        two bytes of the 16-bit draw): three MFMAs into one accumulator on
//        exact fp16 operands (the code, -(4 + hb 2^-8), -(2^-6 + lb 2^-16))
//        against one fp16 query, so the products are exact and only the fp32
//        accumulation rounds.
//   D    lane (n, k) holds tokens 4k..4k+3 of head n: softmax, both meter
//        tiers and the block risk stay lane-local up to 4-lane reductions.
//   PV   O^T[channel][head] += Vhat^T[channel][token] . P^T[token][head]
//        (MFMA 16x16x16 f16, 8 channel tiles); B = P^T is exactly the D layout
//        above (lane (n, k): tokens 4k..4k+3 of head n), so no shuffles; A = the
//        value codes of channel 32 (n / 4) + 4 tile + n % 4, tokens 4k..4k+3,
//        one 32-bit word of the value page layout (dithered INT8: with the
//        draws of the same tokens and channel, read from the key side's LDS
//        tile by 16-bit transpose reads).  Lane (n, k) ends with channels
//        32k..32k+31 of head n.
//   Tier A  a^T[token][head] = W[token][band] . beta[head][band] on two fp32
//        MFMAs 16x16x4.
//   RTN INT8  the code chain alone (no dither); values through 16x16x16 f16
//        MFMAs on the exact code integers, as the fp8 values.
//   16-bit store  keys and values are bf16 (any scheme's output): QK on
//        16x16x32 bf16 MFMAs against the unscaled bf16 query, PV with the
//        attention weights split into bf16 hi + lo halves ([V|V] . [P_hi|P_lo]).
//   Outlier bypass  the exact part of the logits on the bypassed channels,
//        X[token][i] . Q[head][O[i]], on m/4 more fp32 MFMAs 16x16x4; the query
//        operands of the key chains are zero on those channels.
#include <math.h>

#include "wc_common.h"

namespace wc {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// Waves per workgroup (four measured fastest: three and six were slower).
#ifndef WC_DECODE_WAVES
#define WC_DECODE_WAVES 4
#endif
constexpr int kNW = WC_DECODE_WAVES;
constexpr int kThreads = 64 * kNW;
// floats per (b, h, split) partial: m, l, N_A, N_B, o[128], C_A, C_B, N_V, 0
constexpr int kPartial = 136;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i's
// element e is element i % 4 of the four 16-bit values at the address of
// lane 4 e + i / 4.  p: an 8-byte-aligned LDS address.
typedef short s4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 tr16_read(const void* p) {
  const s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(const_cast<void*>(p)));
  return __builtin_bit_cast(uint2, r);
}
__device__ __forceinline__ h2 make_h2(_Float16 a, _Float16 b) { return h2{a, b}; }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// fp16 bit pattern 0x64XX is 1024 + XX exactly; 0xC4XX is -(4 + XX 2^-8) and
// 0xA4XX is -(2^-6 + XX 2^-16): a byte spliced under a fixed exponent.
constexpr uint32_t kMagic = 0x64646464u;
constexpr uint32_t kMagicHiNeg = 0xC4C4C4C4u, kMagicLoNeg = 0xA4A4A4A4u;

// Four INT8 codes stored as offset binary (code + 128, one word) -> two fp16
// pairs of the exact integers: splice under the 1024 exponent, subtract 1152.
__device__ __forceinline__ void codes_to_h(uint32_t u, uint32_t& lo, uint32_t& hi) {
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = as_u32(as_h2(perm(kMagic, u, 0x04010400u)) - bias);
  hi = as_u32(as_h2(perm(kMagic, u, 0x04030402u)) - bias);
}

// Two e4m3fn bytes (byte 0 and 1 of v after the caller's permute) -> fp16
// pair of the exact values: (magnitude << 7 | sign << 8) times 2^8.
__device__ __forceinline__ uint32_t fp8x2_to_h(uint32_t b01) {
  // b01 holds the two bytes in bits 8..15 and 24..31
  const uint32_t mag = (b01 >> 1) & 0x3F803F80u;
  const uint32_t sgn = b01 & 0x80008000u;
  const h2 k256 = {(_Float16)256.0f, (_Float16)256.0f};
  return as_u32(as_h2(mag | sgn) * k256);
}
__device__ __forceinline__ void fp8_to_h(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = fp8x2_to_h(perm(0u, w, 0x010C000Cu));  // bytes: 0, w0, 0, w1
  hi = fp8x2_to_h(perm(0u, w, 0x030C020Cu));  // bytes: 0, w2, 0, w3
}

// Maximum of two finite-or-infinite floats as one v_max_f32: values that
// come out of lane moves would otherwise be re-quieted first (the kernel
// never carries NaNs).
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm volatile("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// max(v, v of lane n ^ 8 within the row) in one DPP instruction; the nop
// covers the wait a DPP read needs after the VALU write of its source.
__device__ __forceinline__ float vmax_ror8(float v) {
  float r;
  asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  return r;
}

// Reductions over the four lanes n, n^16, n^32, n^48 (one head's k groups)
// with the gfx950 row-swap permutes: VALU only, no LDS round trip.  Each swap
// returns the lane's own value and its partner's, in some order.
__device__ __forceinline__ float max4k(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
// Maximum over the whole wave: within each 16-lane row, then across rows.
__device__ __forceinline__ float wave_max64(float v) { return max4k(row16_max(v)); }
__device__ __forceinline__ float sum4k(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Row (16-lane) data movement with DPP: shift by 8 into the upper or lower
// half of every row, or rotate by 8.
__device__ __forceinline__ float dpp_shr8_hi(float old, float src) {   // lanes 8..15 <- lanes 0..7
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), 0x118, 0xF, 0xC, false));
}
__device__ __forceinline__ uint32_t dpp_shl8_lo(uint32_t old, uint32_t src) {   // lanes 0..7 <- lanes 8..15
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x108, 0xF, 0x3, false);
}
__device__ __forceinline__ float dpp_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x128, 0xF, 0xF, false));
}

// Identity move the optimizer cannot see through: a value loaded inside a
// rarely taken branch is consumed there, so the wait for the load is not
// hoisted to the join where every iteration would pay it.
__device__ __forceinline__ int settle(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xE4, 0xF, 0xF, false); }
__device__ __forceinline__ float settle(float v) { return __int_as_float(settle(__float_as_int(v))); }

__device__ __forceinline__ h8 make_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(h8, u);
}
__device__ __forceinline__ h4 make_h4(uint32_t a, uint32_t b) {
  uint2 u = make_uint2(a, b);
  return __builtin_bit_cast(h4, u);
}

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma_bf(uint4 a, uint4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}
// 16x16x16 bf16 (four bf16 per lane and operand)
__device__ __forceinline__ f4 mfma_bf16k(uint2 a, uint2 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0, 0);
}
// Scheme traits: INT8 codes with row scales (dithered or RTN); the 16-bit store.
template <int SCHEME>
constexpr bool int8_codes() {
  return SCHEME == WC_DITHER_INT8 || SCHEME == WC_RTN_INT8;
}
template <int SCHEME>
constexpr int page_bytes() {                  // code bytes of one page-head block, K or V
  return SCHEME == WC_BF16_STORE ? 4096 : 2048;
}

struct DecodeArgs {
  const void* q;
  const int32_t* page_table;
  const int32_t* ctx_len;
  const uint64_t* seed;
  float* partials;
  float* block_logrisk;
  int B, Hq, G, max_pages, n_split, layer;
  unsigned mask;
  float sm_scale;
  float neg_log_dloc;   // -log(delta_loc)
};

// One page of one wave, keys: the lane's 32 key codes of token n, the key
// scales of its tokens, the witness bands 2k, 2k+1 of token n.
struct KLoad {
  uint4 k0, k1, k2, k3;   // k2, k3: the 16-bit store only
  float4 ks;
  float2 w;
  uint2 xo;               // outlier bypass: the lane's bf16 side-store entries
  float4 wv;              // value certificate: the value witnesses of the lane's tokens
  int slot;               // exact-pool slot (-1 = quantized), wave-uniform
};
// Values: 8 channels x 4 tokens of codes and the value scales of the lane's
// tokens.  Both are loaded one page ahead of their use.
struct VLoad {
  uint4 v0, v1, v2, v3;
  float4 vs;
};

// Byte offsets of one lane inside a page-head block (fixed for the kernel):
// the page base is wave-uniform, so every load is a scalar base plus one of
// these 32-bit lane offsets.
// The code layouts put lane l's 16 bytes at 16 l in each 1 KB half of a
// page, so every code load of a wave reads 1 KB in one contiguous run.
struct LaneOff {
  uint32_t k;             // key codes: token n, channels 32k..32k+15 (+1 KB: 32k+16..32k+31)
  uint32_t s;             // scales: tokens 4k (+ r0) onward
  uint32_t w;             // witness bands 2k, 2k+1 of token n (meter off: the key codes again)
  uint32_t v;             // value codes: tiles 0..3 (+1 KB: 4..7) of the lane, tokens 4k..4k+3
  uint32_t o;             // outlier side store: entries k m/4 .. of token n
};

// Buffer resource of one page-head block (raw, untyped, 32-bit data format):
// the base is wave-uniform and lives in SGPRs, accesses past `bytes` read 0.
constexpr int kRsrcFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int64_t off, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(static_cast<const uint8_t*>(base) + off), (short)0,
                                           bytes, kRsrcFlags);
}
// Every page of the cache is read once per decode: the 16-byte code loads
// carry the non-temporal cache policy (2), so they stream through L2 instead
// of displacing lines that are reused.  The 8-byte loads (scales and
// witnesses with the compacted softmax) keep the default policy: one line
// holds several page-heads' entries, read by different workgroups, and a
// streamed line is fetched again for each (8% faster than the default policy
// everywhere on the 32 x 32768 decode, 5% faster than streaming everything).
constexpr int kStream = 2;
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream));
}
__device__ __forceinline__ float2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStream));
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kStream);
}

// With a compacted softmax lane (n, k) evaluates tokens 4k + r0 and
// 4k + r0 + 1 only (r0 = 0 for n < 8, 2 for n >= 8): its scales are a pair.
// The load count and order never depend on run-time flags, and the lane
// offsets stay in fixed registers, so the wait for one page's data never
// waits on the page prefetched after it.
template <int SCHEME, bool PAIR, int NO4, bool MV>
__device__ __forceinline__ void load_page(const wc_cache& c, int64_t pg, const LaneOff& lo, bool meterA, KLoad& d,
                                          VLoad& e) {
  if (MV) {                                    // value witnesses: 16 floats per page-head block
    const __amdgpu_buffer_rsrc_t wvr = page_rsrc(c.v_witness, pg * 64, 64);
    if (PAIR) {
      const float2 t = bload8(wvr, lo.s);
      d.wv = make_float4(t.x, t.y, 0.f, 0.f);
    } else {
      d.wv = __builtin_bit_cast(float4, bload16(wvr, lo.s));
    }
  }
  if (NO4 > 0) {                               // side store: 32 m bytes per page-head block
    const __amdgpu_buffer_rsrc_t orr = page_rsrc(c.k_outlier, pg * (128 * NO4), 128 * NO4);
    if (NO4 == 4)
      d.xo = __builtin_bit_cast(uint2, bload8(orr, lo.o));
    else
      d.xo = make_uint2(bload4(orr, lo.o), 0u);
  }
  constexpr int PB = page_bytes<SCHEME>();
  const __amdgpu_buffer_rsrc_t kr = page_rsrc(c.k_codes, pg * PB, PB);
  const __amdgpu_buffer_rsrc_t vr = page_rsrc(c.v_codes, pg * PB, PB);
  const __amdgpu_buffer_rsrc_t wr = meterA ? page_rsrc(c.witness, pg * 512, 512) : kr;
  d.k0 = bload16(kr, lo.k);
  d.k1 = bload16(kr, lo.k + 1024);
  if (SCHEME == WC_BF16_STORE) {
    d.k2 = bload16(kr, lo.k + 2048);
    d.k3 = bload16(kr, lo.k + 3072);
  }
  d.w = bload8(wr, lo.w);
  e.v0 = bload16(vr, lo.v);
  e.v1 = bload16(vr, lo.v + 1024);
  if (SCHEME == WC_BF16_STORE) {
    e.v2 = bload16(vr, lo.v + 2048);
    e.v3 = bload16(vr, lo.v + 3072);
  }
  if (int8_codes<SCHEME>()) {
    const __amdgpu_buffer_rsrc_t ksr = page_rsrc(c.k_scale, pg * 64, 64);
    const __amdgpu_buffer_rsrc_t vsr = page_rsrc(c.v_scale, pg * 64, 64);
    if (PAIR) {
      const float2 t = bload8(ksr, lo.s), u = bload8(vsr, lo.s);
      d.ks = make_float4(t.x, t.y, 0.f, 0.f);
      e.vs = make_float4(u.x, u.y, 0.f, 0.f);
    } else {
      d.ks = __builtin_bit_cast(float4, bload16(ksr, lo.s));
      e.vs = __builtin_bit_cast(float4, bload16(vsr, lo.s));
    }
  } else {
    d.ks = make_float4(1.f, 1.f, 1.f, 1.f);
    e.vs = make_float4(1.f, 1.f, 1.f, 1.f);
  }
}

// When a layer's arrays are under 4 GB, one resource per array and layer
// serves every page: the page enters as a 32-bit scalar offset, which saves
// the per-page resource set-up.
struct LayerBufs {
  __amdgpu_buffer_rsrc_t k, v, w, ks, vs, o, wv;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t layer_rsrc(const void* base, int64_t off, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(static_cast<const uint8_t*>(base) + off), (short)0,
                                           (int)(uint32_t)bytes, kRsrcFlags);
}
__device__ __forceinline__ uint4 bload16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kStream));
}
__device__ __forceinline__ float2 bload8s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
__device__ __forceinline__ uint32_t bload4s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, kStream);
}
// pg: page-head block index within the layer (phys * Hkv + g)
template <int SCHEME, bool PAIR, int NO4, bool MV>
__device__ __forceinline__ void load_page_soff(const LayerBufs& lb, uint32_t pg, const LaneOff& lo, bool meterA,
                                               KLoad& d, VLoad& e) {
  if (MV) {
    if (PAIR) {
      const float2 t = bload8s(lb.wv, lo.s, pg * 64u);
      d.wv = make_float4(t.x, t.y, 0.f, 0.f);
    } else {
      d.wv = __builtin_bit_cast(float4, bload16s(lb.wv, lo.s, pg * 64u));
    }
  }
  if (NO4 > 0) {
    if (NO4 == 4)
      d.xo = __builtin_bit_cast(uint2, bload8s(lb.o, lo.o, pg * (128u * NO4)));
    else
      d.xo = make_uint2(bload4s(lb.o, lo.o, pg * (128u * NO4)), 0u);
  }
  constexpr uint32_t PB = page_bytes<SCHEME>();
  d.k0 = bload16s(lb.k, lo.k, pg * PB);
  d.k1 = bload16s(lb.k, lo.k + 1024, pg * PB);
  if (SCHEME == WC_BF16_STORE) {
    d.k2 = bload16s(lb.k, lo.k + 2048, pg * PB);
    d.k3 = bload16s(lb.k, lo.k + 3072, pg * PB);
  }
  d.w = bload8s(lb.w, lo.w, meterA ? pg * 512u : pg * PB);
  e.v0 = bload16s(lb.v, lo.v, pg * PB);
  e.v1 = bload16s(lb.v, lo.v + 1024, pg * PB);
  if (SCHEME == WC_BF16_STORE) {
    e.v2 = bload16s(lb.v, lo.v + 2048, pg * PB);
    e.v3 = bload16s(lb.v, lo.v + 3072, pg * PB);
  }
  if (int8_codes<SCHEME>()) {
    if (PAIR) {
      const float2 t = bload8s(lb.ks, lo.s, pg * 64u), u = bload8s(lb.vs, lo.s, pg * 64u);
      d.ks = make_float4(t.x, t.y, 0.f, 0.f);
      e.vs = make_float4(u.x, u.y, 0.f, 0.f);
    } else {
      d.ks = __builtin_bit_cast(float4, bload16s(lb.ks, lo.s, pg * 64u));
      e.vs = __builtin_bit_cast(float4, bload16s(lb.vs, lo.s, pg * 64u));
    }
  } else {
    d.ks = make_float4(1.f, 1.f, 1.f, 1.f);
    e.vs = make_float4(1.f, 1.f, 1.f, 1.f);
  }
}

// expm1 for c >= 0: series below 2^-5, else 2^(c log2 e) - 1 on v_exp_f32.
__device__ __forceinline__ float expm1_fast(float c) {
  const float e = __builtin_amdgcn_exp2f(c * kLog2e) - 1.0f;
  const float p = fmaf(c * c, fmaf(c, fmaf(c, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f), c);
  return c < 0.03125f ? p : e;
}

// p (e^c - 1) for a bound c in [0, 1/4): p c (1 + c/2 + c^2/6 + c^3/24 +
// c^4/120 + c^5/720), whose truncation error is below c^6/5040 < 5e-8
// relative, under the fp32 rounding; no exp and no cancellation.
__device__ __forceinline__ float p_expm1_small(float p, float c) {
  const float t = fmaf(c, fmaf(c, fmaf(c, fmaf(c, fmaf(c, 1.0f / 720.0f, 1.0f / 120.0f), 1.0f / 24.0f), 1.0f / 6.0f),
                                0.5f), 1.0f);
  return (p * c) * t;
}

__device__ __forceinline__ f4 mfma_f32(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Lazy rescale: the running max of a head only moves when a page's max
// exceeds it by more than 8 (log2 units), so exp2 weights stay <= 256.
constexpr float kRescaleSlack = 8.0f;

// Pages each wave keeps in flight ahead of the one it processes.
#ifndef WC_PREFETCH_DEPTH
#define WC_PREFETCH_DEPTH 1
#endif
constexpr int kDepth = WC_PREFETCH_DEPTH;

// Waves per SIMD the register allocation must allow: three for bf16 queries
// (168 registers, no spills), two for fp32 queries (their split query
// operand needs more).
#ifndef WC_DECODE_MIN_BLOCKS_BF16
#define WC_DECODE_MIN_BLOCKS_BF16 3
#endif
#ifndef WC_DECODE_MIN_BLOCKS_OUTL
#define WC_DECODE_MIN_BLOCKS_OUTL 3
#endif
// The 16-bit store keeps twice the bytes of a page in flight: two waves.
template <int SCHEME, bool QF32, int NO4>
constexpr int decode_waves_per_simd() {
  return (QF32 || SCHEME == WC_BF16_STORE) ? 2 : NO4 > 0 ? WC_DECODE_MIN_BLOCKS_OUTL : WC_DECODE_MIN_BLOCKS_BF16;
}

// CMP: the query group has at most 8 heads, so the softmax and meter run
// compacted on two tokens per lane (lanes n + 8 take tokens 2, 3 of head n).
// NO4: outlier bypass with m = 4 NO4 exact key channels (0 = none).
// MV: the value certificate (reads the value witnesses).
// MODE: the meter configuration fixed at compile time (kModeRuntime: read
// from the arguments), so the common launches carry no flag tests.
constexpr int kModeRuntime = 0, kModeOff = 1, kModeOn = 2;
template <int SCHEME, bool QF32, bool CMP, bool SOFF, int NO4, bool MV, int MODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<SCHEME, QF32, NO4>())))
decode_kernel(wc_cache c, DecodeArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int G = a.G;
  const int h = g * G + n;                     // query head of lane column n
  const bool hv = n < G;
  const int S = a.ctx_len[b];
  const int P = (S + 15) >> 4;
  const int p0 = (int)((int64_t)split * P / a.n_split), p1 = (int)((int64_t)(split + 1) * P / a.n_split);
  // fixed modes: off; Tier A (+ B for dithered INT8)
  const bool meterA = MODE == kModeRuntime ? (a.mask & WC_METER_A) != 0 : MODE != kModeOff;
  const bool meterB = SCHEME == WC_DITHER_INT8 &&
                      (MODE == kModeRuntime ? (a.mask & WC_METER_B) != 0 : MODE != kModeOff);
  // (the block output stays a run-time test: with it fixed, the compiler's
  // schedule of the risk path needs more registers than three waves per SIMD
  // allow, and spills)
  const bool risk = a.block_logrisk != nullptr;
  const bool riskmax = MODE == kModeRuntime && (a.mask & WC_BLOCK_CMAX) != 0;   // block output: max c, not log risk

  // ---------------------------------------------------------------- query prep
  // lane (n, k) holds channels 32k..32k+31 of head n.
  // (the query's words are requested first and converted after the first
  // page-table batch and page are requested, so that the latencies overlap)
  uint4 qw[8];
  if (hv) {
    const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.q) +
                                                     (((int64_t)b * a.Hq + h) * 128 + 32 * kq) * (QF32 ? 4 : 2));
#pragma unroll
    for (int i = 0; i < (QF32 ? 8 : 4); ++i) qw[i] = qp[i];
  }
  const int r0 = CMP ? 2 * (n >> 3) : 0;
  LaneOff lo;
  lo.k = (uint32_t)(16 * lane);
  lo.s = (uint32_t)(4 * (4 * kq + r0));
  lo.w = meterA ? (uint32_t)(4 * (8 * n + 2 * kq)) : lo.k;
  lo.v = (uint32_t)(16 * lane);
  lo.o = (uint32_t)(2 * NO4 * (4 * n + kq));
  // Each wave takes a contiguous quarter of the split's pages: page i of
  // this wave is page w0 + i.  Its physical page and exact-pool slot come
  // from lane i % 64 of a batch read once per 64 pages, so the loop never
  // waits on a page-table read.  The first batch and page are requested
  // before the query is prepared, so that their latency overlaps it.
  const int per = (p1 - p0 + kNW - 1) / kNW;
  const int w0 = p0 + wave * per;
  const int npw = max(0, min(p1, w0 + per) - w0);
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
  const int64_t pg_base = (int64_t)a.layer * c.num_pages;
  LayerBufs lb;
  if (SOFF) {
    const int64_t lph = c.num_pages * c.num_kv_heads;     // page-head blocks per layer
    const int64_t l0 = (int64_t)a.layer * lph;
    constexpr int64_t PB = page_bytes<SCHEME>();
    lb.k = layer_rsrc(c.k_codes, l0 * PB, (uint64_t)lph * PB);
    lb.v = layer_rsrc(c.v_codes, l0 * PB, (uint64_t)lph * PB);
    lb.w = meterA ? layer_rsrc(c.witness, l0 * 512, (uint64_t)lph * 512) : lb.k;
    lb.o = lb.ks = lb.vs = lb.wv = lb.k;       // (unused unless set below)
    if (MV) lb.wv = layer_rsrc(c.v_witness, l0 * 64, (uint64_t)lph * 64);
    if (NO4 > 0) lb.o = layer_rsrc(c.k_outlier, l0 * (128 * NO4), (uint64_t)lph * (128 * NO4));
    if (int8_codes<SCHEME>()) {
      lb.ks = layer_rsrc(c.k_scale, l0 * 64, (uint64_t)lph * 64);
      lb.vs = layer_rsrc(c.v_scale, l0 * 64, (uint64_t)lph * 64);
    }
  }
  int bphys = 0, bslot = -1;
  auto batch = [&](int i0) {
    const int i = i0 + lane;
    const int ph = i < npw ? ptab[w0 + i] : 0;
    bphys = settle(ph);                        // the page loads wait for these, in this rare branch
    // the slots are gathered next to the page loads; with one page in
    // flight they are read when the page is processed, so the first page's
    // loads do not wait for them
    const int sl = (i < npw && c.exact_slot) ? c.exact_slot[(pg_base + ph) * c.num_kv_heads + g] : -1;
    bslot = kDepth == 1 ? sl : settle(sl);
  };
  // Past the wave's last page the prefetch requests physical page 0 of the
  // layer: the loads (and so every wait) are the same as for a real page, the
  // data is never used, and the block, requested by every wave, stays in L2
  // instead of a last page being read from HBM a second time.
  auto fetch = [&](int i, KLoad& d, VLoad& e) {
    const bool past = i >= npw;
    if (!past && (i & 63) == 0) batch(i);
    const int phys = past ? 0 : __builtin_amdgcn_readlane(bphys, i & 63);
    if (kDepth > 1) d.slot = past ? -1 : __builtin_amdgcn_readlane(bslot, i & 63);
    if (SOFF)
      load_page_soff<SCHEME, CMP, NO4, MV>(lb, (uint32_t)(phys * c.num_kv_heads + g), lo, meterA, d, e);
    else
      load_page<SCHEME, CMP, NO4, MV>(c, (pg_base + phys) * c.num_kv_heads + g, lo, meterA, d, e);
  };
  KLoad kA, kB;
  VLoad vA, vB;
  // (also with no page: the batch of a wave without pages reads no table and
  // requests physical page 0, in bounds and unused, and every path then
  // waits for the query words here)
  if (kDepth == 1) {
    batch(0);
    const int phys = __builtin_amdgcn_readlane(bphys, 0);
    if (SOFF)
      load_page_soff<SCHEME, CMP, NO4, MV>(lb, (uint32_t)(phys * c.num_kv_heads + g), lo, meterA, kA, vA);
    else
      load_page<SCHEME, CMP, NO4, MV>(c, (pg_base + phys) * c.num_kv_heads + g, lo, meterA, kA, vA);
  }
  float qf[32];
  if (hv) {
    if (QF32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qf[4 * i] = __uint_as_float(qw[i].x); qf[4 * i + 1] = __uint_as_float(qw[i].y);
        qf[4 * i + 2] = __uint_as_float(qw[i].z); qf[4 * i + 3] = __uint_as_float(qw[i].w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {qw[i].x, qw[i].y, qw[i].z, qw[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[8 * i + 2 * e] = __uint_as_float(w[e] << 16);
          qf[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) qf[i] = 0.0f;
  }
  // The query of head n as bf16 pieces for repaired blocks (exact bf16 keys
  // on bf16 MFMAs): one piece for a bf16 query, three that sum exactly to an
  // fp32 one.  Staged in LDS once per workgroup (rows padded to 17 slots, so
  // the 16 lanes of one read hit distinct banks); the repaired branch reads
  // them per MFMA.
  constexpr int NQP = QF32 ? 3 : 1;
  __shared__ __align__(16) uint4 sQ[NQP][16][17];
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t pc[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a0 = __float_as_uint(qf[8 * j + 2 * e]), a1 = __float_as_uint(qf[8 * j + 2 * e + 1]);
        const uint32_t h0 = a0 & 0xFFFF0000u, h1 = a1 & 0xFFFF0000u;
        pc[0][e] = (h0 >> 16) | h1;
        if (QF32) {
          const float r0 = __uint_as_float(a0) - __uint_as_float(h0), r1 = __uint_as_float(a1) - __uint_as_float(h1);
          const uint32_t m0 = __float_as_uint(r0) & 0xFFFF0000u, m1 = __float_as_uint(r1) & 0xFFFF0000u;
          const uint32_t l0 = __float_as_uint(r0 - __uint_as_float(m0));
          const uint32_t l1 = __float_as_uint(r1 - __uint_as_float(m1));
          pc[1][e] = (m0 >> 16) | m1;
          pc[2][e] = (l0 >> 16) | (l1 & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int pq = 0; pq < NQP; ++pq) sQ[pq][n][4 * kq + j] = make_uint4(pc[pq][0], pc[pq][1], pc[pq][2], pc[pq][3]);
    }
  }
  __syncthreads();
  float qmax = 0.0f, bsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 32; ++i) bsum[i >> 3] = fmaf(qf[i], qf[i], bsum[i >> 3]);   // Tier A: the full query
  // Outlier bypass: the key chains see the query with the bypassed channels
  // zeroed; entry k m/4 + j of the side store (channel O[k m/4 + j]) meets
  // head n's query there.  m = 16 with a bf16 query (BFO): bOq holds those
  // four query entries as bf16, K slots 4k..4k+3 of one 16x16x16 bf16 MFMA,
  // so every product is exact and the scale sm log2 e is applied once to the
  // sum.  Otherwise fp32 MFMA j takes bO[j] = q[O[k m/4 + j]] sm log2 e (for
  // m = 8 the bf16 form would need a zero register per page buffer, past the
  // register limit).
  constexpr bool BFO = NO4 == 4 && !QF32;
  float bO[4] = {0.f, 0.f, 0.f, 0.f};
  uint2 bOq = make_uint2(0u, 0u);
  const float osc = a.sm_scale * kLog2e;
  float qz2 = 0.0f;                            // sum of q^2 off the bypassed channels (Tier B)
  if (NO4 > 0) {
    const int32_t* oc = c.outlier_ch + ((int64_t)a.layer * c.num_kv_heads + g) * (4 * NO4);
    uint32_t omask = 0;
#pragma unroll
    for (int e = 0; e < 4 * NO4; ++e) {
      const int ch = oc[e] & 127;
      omask |= (ch >> 5) == kq ? 1u << (ch & 31) : 0u;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      qf[i] = ((omask >> i) & 1u) ? 0.0f : qf[i];
      qz2 = fmaf(qf[i], qf[i], qz2);
    }
    qz2 += shfl_xor(qz2, 16);
    qz2 += shfl_xor(qz2, 32);
    if (hv) {
      const int64_t qrow = ((int64_t)b * a.Hq + h) * 128;
#pragma unroll
      for (int j = 0; j < NO4; ++j) {
        const int ch = oc[kq * NO4 + j] & 127;
        if (BFO) {
          const uint32_t qb = reinterpret_cast<const uint16_t*>(a.q)[qrow + ch];
          if (j == 0) bOq.x |= qb;
          if (j == 1) bOq.x |= qb << 16;
          if (j == 2) bOq.y |= qb;
          if (j == 3) bOq.y |= qb << 16;
        } else {
          const float qv = QF32 ? reinterpret_cast<const float*>(a.q)[qrow + ch]
                                : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qrow + ch]);
          bO[j] = qv * osc;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) qmax = fmaxf(qmax, fabsf(qf[i]));
  qmax = fmaxf(qmax, shfl_xor(qmax, 16));
  qmax = fmaxf(qmax, shfl_xor(qmax, 32));
  int qe = 0;
  if (qmax > 0.0f) {
    int ex;
    frexpf(qmax, &ex);                        // qmax in [2^(ex-1), 2^ex)
    qe = 15 - ex;                              // scaled max in [2^14, 2^15): exact in fp16 for bf16 q
  }
  h8 Qhi[4], Qlo[4];
  float qsum = 0.0f;                           // sum of the fp16 query operand (dither bias)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x0 = ldexpf(qf[8 * j + 2 * e], qe), x1 = ldexpf(qf[8 * j + 2 * e + 1], qe);
      _Float16 a0 = (_Float16)x0, a1 = (_Float16)x1;
      h2 hv2 = {a0, a1};
      hw[e] = as_u32(hv2);
      qsum += (float)a0 + (float)a1;
      if (QF32) {
        _Float16 b0 = (_Float16)(x0 - (float)a0), b1 = (_Float16)(x1 - (float)a1);
        h2 lv2 = {b0, b1};
        lw[e] = as_u32(lv2);
        qsum += (float)b0 + (float)b1;
      }
    }
    Qhi[j] = make_h8(hw[0], hw[1], hw[2], hw[3]);
    if (QF32) Qlo[j] = make_h8(lw[0], lw[1], lw[2], lw[3]);
  }
  qsum += shfl_xor(qsum, 16);
  qsum += shfl_xor(qsum, 32);
  // 16-bit store: the unscaled query as bf16 (exact for bf16 q; fp32 q adds
  // the bf16 of the remainder as a second operand)
  uint4 Qb[4], Qbl[4];
  if (SCHEME == WC_BF16_STORE) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u0 = __float_as_uint(qf[8 * j + 2 * e]) & 0xFFFF0000u;
        const uint32_t u1 = __float_as_uint(qf[8 * j + 2 * e + 1]) & 0xFFFF0000u;
        hw[e] = (u0 >> 16) | u1;
        if (QF32) {
          const uint32_t r0 = __float_as_uint(qf[8 * j + 2 * e] - __uint_as_float(u0));
          const uint32_t r1 = __float_as_uint(qf[8 * j + 2 * e + 1] - __uint_as_float(u1));
          lw[e] = (r0 >> 16) | (r1 & 0xFFFF0000u);
        }
      }
      Qb[j] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      if (QF32) Qbl[j] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
  // the store's keys are unscaled: their pages use the token factor 2^qe
  // (with the compacted softmax, lanes n + 8 take head n's)
  float store_st = ldexpf(1.0f, qe);
  if (CMP) store_st = dpp_shr8_hi(store_st, store_st);
  // band norms: lane k holds bands (4k + jj) mod 8 of one half; halves are k, k^2
  float bfull[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) bfull[jj] = bsum[jj] + shfl_xor(bsum[jj], 32);
  float qn2 = bfull[0] + bfull[1] + bfull[2] + bfull[3];
  qn2 += shfl_xor(qn2, 16);                    // ||q_h||^2 over all 8 bands
  float beta[8];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float mine = a.sm_scale * sqrtf(bfull[jj]);
    float other = shfl_xor(mine, 16);
    beta[jj] = (kq & 1) ? other : mine;        // k even holds bands 0..3, odd 4..7
    beta[4 + jj] = (kq & 1) ? mine : other;
  }
  // Tier A operands of the two fp32 MFMAs: K slot k <-> bands 2k and 2k+1
  // (selects, not an index by the lane's k: that would go through scratch)
  const float b2k = kq == 0 ? beta[0] : kq == 1 ? beta[2] : kq == 2 ? beta[4] : beta[6];
  const float b2k1 = kq == 0 ? beta[1] : kq == 1 ? beta[3] : kq == 2 ? beta[5] : beta[7];
  const float bA0 = hv ? b2k : 0.0f, bA1 = hv ? b2k1 : 0.0f;
  const float qs2 = a.sm_scale * kLog2e * ldexpf(1.0f, -qe);     // log2-unit logit per raw unit
  // the dither bytes enter the key MFMAs as -(4 + hb 2^-8) and
  // -(2^-6 + lb 2^-16); with xi = hb 2^-8 + lb 2^-16 - 1/2 the chain's start
  // value qsum (4.5 + 2^-6) leaves sum q' (code - xi)
  const float qbias = qsum * 4.515625f;
  const f4 kb4 = SCHEME == WC_DITHER_INT8 ? f4{qbias, qbias, qbias, qbias} : f4{0.f, 0.f, 0.f, 0.f};
  const float logterm = logf(2.0f * (float)S) + a.neg_log_dloc;
  const float kappa = a.sm_scale * sqrtf(NO4 > 0 ? qz2 : qn2) * sqrtf(fmaxf(logterm, 0.0f) / 6.0f);

  const uint32_t key = SCHEME == WC_DITHER_INT8 ? stream_key(a.seed[b], (uint32_t)a.layer, (uint32_t)g) : 0u;
  // LCG state of the lane's first counter on logical page 0, key + 64 n + 16 k
  // (page jj adds 1024 jj counters: a wave-uniform constant times kPcgMul)
  const uint32_t st_lane = (key + (uint32_t)(64 * n + 16 * kq)) * kPcgMul + kPcgInc;
  // compacted softmax: lane (n, k) evaluates head n & 7, tokens 4k + r0, +1
  constexpr int NV = CMP ? 2 : 4;
  const float qs2c = CMP ? dpp_shr8_hi(qs2, qs2) : qs2;
  const float kappac = CMP ? dpp_shr8_hi(kappa, kappa) : kappa;
  // Per-wave LDS tile of the page's dither high bytes as fp16 operands
  // -(4 + byte 2^-8): the key side (lane = token) hashes each draw once and
  // stores [token][8-channel group]; the value side (lane = channel group)
  // reads four tokens back.  Rows are padded to 17 slots so that neither
  // side's 16 lanes of one instruction share a bank.  The space is the
  // end-of-split combine buffer.
  __shared__ __align__(16) uint4 smem[kNW * 2 * 16 * 16];
  uint4 (*sH)[17] = reinterpret_cast<uint4 (*)[17]>(smem + wave * 16 * 17);
  __shared__ float sRisk[kNW][16][16];
  float (*sR)[16] = sRisk[wave];

  // ---------------------------------------------------------------- state
  // m_ref: the running max of the logits (log2 units) minus sig, the
  // value-range offset (INT8 caches; 0 otherwise); sv_ref: the largest value
  // scale seen so far (wave-uniform)
  float m_ref = -INFINITY, l_run = 0.0f, na = 0.0f, nb = 0.0f;
  float sig = 0.0f, sv_ref = 0.0f;
  float m_lim = -INFINITY;                     // the running max plus the rescale slack
  float ca_max = 0.0f, cb_max = 0.0f;          // largest per-token bound of each tier (tanh bound)
  float nvv = 0.0f;                            // value certificate: sum 2^(l2 - m) ||v^ - v||
  f4 O[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) O[t] = f4{0.f, 0.f, 0.f, 0.f};

  // one page of this wave; the loop below alternates two prefetch buffers
  const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
  float vsum = 0.0f;                           // sum of the value weights p s fed to the MFMA
  auto page = [&](const KLoad& cur, const VLoad& vl, KLoad& nxt, VLoad& vnxt, const int i) {
    // the page kDepth ahead; past the end the last page loads itself again
    // so that every iteration issues the same loads
    // (its exact-pool slot first: the prefetch below may start the next batch)
    const int slot = kDepth == 1 ? __builtin_amdgcn_readlane(bslot, i & 63) : cur.slot;
    fetch(i + kDepth, nxt, vnxt);
    const int jj = w0 + i;
    const int tok0 = jj * 16;
    const bool exact = slot >= 0;              // wave-uniform
    const bool full = tok0 + 16 <= S;          // wave-uniform: only the last page is ragged

    // ---------------- Tier A: a^T = W . beta^T on two fp32 MFMAs, issued first
    // so that their latency hides behind the key work (zeroed below for a
    // repaired block)
    f4 Da = zero4;
    if (meterA) Da = mfma_f32(cur.w.y, bA1, mfma_f32(cur.w.x, bA0, zero4));
    // exact logits on the bypassed channels (log2 units; BFO: the sum of the
    // exact products, scaled where the logit is formed), also for repaired
    // blocks: their pool keys meet the zeroed query
    f4 Do = zero4;
    if (BFO) Do = mfma_bf16k(cur.xo, bOq, Do);
    if (NO4 > 0 && !BFO) {
      Do = mfma_f32(__uint_as_float(cur.xo.x << 16), bO[0], Do);
      Do = mfma_f32(__uint_as_float(cur.xo.x & 0xFFFF0000u), bO[1], Do);
      if (NO4 == 4) {
        Do = mfma_f32(__uint_as_float(cur.xo.y << 16), bO[2], Do);
        Do = mfma_f32(__uint_as_float(cur.xo.y & 0xFFFF0000u), bO[3], Do);
      }
    }

    // ---------------- QK^T: three MFMA chains over 128 channels
    f4 Dc = zero4;
    float st[4] = {cur.ks.x, cur.ks.y, cur.ks.z, cur.ks.w};
    const uint32_t kw[8] = {cur.k0.x, cur.k0.y, cur.k0.z, cur.k0.w, cur.k1.x, cur.k1.y, cur.k1.z, cur.k1.w};
    // LCG state of the lane's first counter, key + 64 token + 16 k; the
    // other 15 counters are consecutive (their states differ by constants)
    const uint32_t st0 = st_lane + (uint32_t)jj * (1024u * kPcgMul);
    // draws of token n, channels 32k + 8j .. +7, as fp16 pairs -(4 + hb 2^-8)
    // and -(2^-6 + lb 2^-16) of the high and low byte; the high ones are
    // published to LDS for the values
    auto draws = [&](int j, uint32_t (&hh)[4], uint32_t (&ll)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t wd = pcg_out_sdwa(st0 + (uint32_t)(4 * j + e) * kPcgMul);
        hh[e] = perm(kMagicHiNeg, wd, 0x04030401u);
        ll[e] = perm(kMagicLoNeg, wd, 0x04020400u);
      }
      sH[n][4 * kq + j] = make_uint4(hh[0], hh[1], hh[2], hh[3]);
    };
    if (!exact && SCHEME == WC_BF16_STORE) {
      const uint4 kx[4] = {cur.k0, cur.k1, cur.k2, cur.k3};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Dc = mfma_bf(kx[j], Qb[j], j == 0 ? zero4 : Dc);
        if (QF32) Dc = mfma_bf(kx[j], Qbl[j], Dc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) st[r] = store_st;
    } else if (!exact) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t hh[4], ll[4], c0, c1, c2, c3;
        if (SCHEME == WC_DITHER_INT8) {
          draws(j, hh, ll);
          codes_to_h(kw[2 * j], c0, c1);
          codes_to_h(kw[2 * j + 1], c2, c3);
        } else if (SCHEME == WC_RTN_INT8) {
          codes_to_h(kw[2 * j], c0, c1);
          codes_to_h(kw[2 * j + 1], c2, c3);
        } else {
          fp8_to_h(kw[2 * j], c0, c1);
          fp8_to_h(kw[2 * j + 1], c2, c3);
        }
        const h8 Ac = make_h8(c0, c1, c2, c3);
        // the chain starts from the cancellation of the byte offsets (INT8)
        Dc = mfma32(Ac, Qhi[j], j == 0 ? kb4 : Dc);
        if (QF32) Dc = mfma32(Ac, Qlo[j], Dc);
        if (SCHEME == WC_DITHER_INT8) {
          const h8 Ah = make_h8(hh[0], hh[1], hh[2], hh[3]);
          const h8 Al = make_h8(ll[0], ll[1], ll[2], ll[3]);
          Dc = mfma32(Ah, Qhi[j], Dc);
          Dc = mfma32(Al, Qhi[j], Dc);
          if (QF32) {
            Dc = mfma32(Ah, Qlo[j], Dc);
            Dc = mfma32(Al, Qlo[j], Dc);
          }
        }
      }
    } else {
      // repaired block: the exact bf16 keys of token n (channels 32k..32k+31)
      // from the pool against head n's unscaled query pieces on bf16 MFMAs,
      // so every product is exact.  The full query meets the full exact key
      // (the outlier bypass's side-store logits are not added here).  The
      // values still need the draws.  The pool loads are issued before the
      // hashing so that their latency overlaps it.
      // (a wave-uniform base, the slot's 4 KB, plus the lane offset 256 n + 64 k)
      const uint8_t* pb = reinterpret_cast<const uint8_t*>(c.exact_pool) + (int64_t)slot * 4096;
      const uint32_t po = (uint32_t)(256 * n + 64 * kq);
      uint4 xv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = *reinterpret_cast<const uint4*>(pb + po + 16 * j);
      if (SCHEME == WC_DITHER_INT8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t hh[4], ll[4];
          draws(j, hh, ll);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int pq = 0; pq < NQP; ++pq) Dc = mfma_bf(xv[j], sQ[pq][n][4 * kq + j], (j == 0 && pq == 0) ? zero4 : Dc);
      }
      // the unscaled query: the token factor 2^qe cancels the logit scale's 2^-qe
#pragma unroll
      for (int r = 0; r < 4; ++r) st[r] = store_st;
      Da = zero4;
      Do = zero4;
    }
    // the value side's draws: tile t of lane (n, k) is channel
    // 32 (n / 4) + 4 t + n % 4 (the value page layout), tokens 4k..4k+3.  The
    // 16-bit transpose read gives lane n of each 16-lane group element n % 4
    // of the four halves addressed by lane 4 e + n / 4, as its element e; so
    // lane n addresses token 4k + n / 4, channels 32 (n % 4) + 4 t onward, and
    // receives the four tokens' operands of its channel, in token order.
    if (SCHEME == WC_DITHER_INT8) __builtin_amdgcn_wave_barrier();
    // raw = sum q' (code - xi) (a repaired block: sum q' k of the exact keys)
    float raw[4] = {Dc[0], Dc[1], Dc[2], Dc[3]};
    float cA[4] = {Da[0], Da[1], Da[2], Da[3]};
    float lo2[4] = {Do[0], Do[1], Do[2], Do[3]};
    if (CMP) {                                 // lanes n + 8 take tokens 2, 3 of head n
      raw[0] = dpp_shr8_hi(raw[0], raw[2]);
      raw[1] = dpp_shr8_hi(raw[1], raw[3]);
      cA[0] = dpp_shr8_hi(cA[0], cA[2]);
      cA[1] = dpp_shr8_hi(cA[1], cA[3]);
      if (NO4 > 0) {
        lo2[0] = dpp_shr8_hi(lo2[0], lo2[2]);
        lo2[1] = dpp_shr8_hi(lo2[1], lo2[3]);
      }
    }
    float l2[4], cB[4];
    const float kapB = (meterB && !exact) ? kappac : 0.0f;
    float sv[4] = {vl.vs.x, vl.vs.y, vl.vs.z, vl.vs.w};
    float wvv[4] = {cur.wv.x, cur.wv.y, cur.wv.z, cur.wv.w};
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      l2[r] = qs2c * st[r] * raw[r];
      if (NO4 > 0) l2[r] = BFO ? fmaf(lo2[r], osc, l2[r]) : l2[r] + lo2[r];
      cB[r] = kapB * st[r];
    }
    if (!full) {                               // tokens past the end: no weight, no bound, finite scales
#pragma unroll
      for (int r = 0; r < NV; ++r) {
        const bool ok = tok0 + 4 * kq + r0 + r < S;
        l2[r] = ok ? l2[r] : -INFINITY;
        cA[r] = ok ? cA[r] : 0.0f;
        cB[r] = ok ? cB[r] : 0.0f;
        sv[r] = ok ? sv[r] : 0.0f;
        if (MV) wvv[r] = ok ? wvv[r] : 0.0f;
      }
    }

    // ---------------- online softmax with lazy rescale
    // Each lane tests its own tokens; only when some lane needs it does the
    // head's maximum get reduced (a head's lanes always agree on m_ref).
    float lmax = vmax(l2[0], l2[1]);
    float svmax = vmax(sv[0], sv[1]);
    if (!CMP) {
      lmax = vmax(lmax, vmax(l2[2], l2[3]));
      svmax = vmax(svmax, vmax(sv[2], sv[3]));
    }
    // (bitwise, so that the test compiles to compares and mask logic, not branches)
    // (a value scale above the largest seen so far also rescales: the
    // weights p s_v fed to the fp16 PV operand are kept in range by taking
    // m_ref = the running max minus sig, with the wave-uniform sig chosen so
    // that s_max 2^sig lies in [64, 128): then p s_v < 2^8 2^7 and the
    // weights of the largest scales stay far above fp16's subnormals.  Every
    // sum is taken relative to m_ref, so sig cancels in o, LSE and the meters.)
    const bool need_m = lmax > m_lim;
    const bool need = int8_codes<SCHEME>() ? need_m | (svmax > sv_ref) : need_m;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      float tmax = lmax, anyn = need_m ? 1.0f : 0.0f;
      if (CMP) {
        tmax = vmax_ror8(tmax);
        anyn = vmax_ror8(anyn);
      }
      tmax = max4k(tmax);
      anyn = max4k(anyn);
      float m_new = anyn > 0.0f ? tmax - sig : m_ref;
      if (int8_codes<SCHEME>()) {
        const float smax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max64(svmax))));
        if (smax > sv_ref) {
          int e;
          frexpf(smax, &e);                    // smax in [2^(e-1), 2^e): 2^(7-e) smax in [64, 128)
          const float sig_new = (float)(7 - e);
          m_new += sig - sig_new;              // the same running max, the new offset
          sig = sig_new;
          sv_ref = smax;
        }
      }
      const float alpha = m_ref == -INFINITY ? 0.0f : exp2f(m_ref - m_new);
      l_run *= alpha;
      na *= alpha;
      if (MV) nvv *= alpha;
      nb *= alpha;
      vsum *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) O[t] *= alpha;
      m_ref = m_new;
      m_lim = m_new + sig + kRescaleSlack;
    }
    float p[4], dl[4];
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      dl[r] = l2[r] - m_ref;
      p[r] = __builtin_amdgcn_exp2f(dl[r]);
    }
    float psum = p[0];
#pragma unroll
    for (int r = 1; r < NV; ++r) psum += p[r];
    l_run += psum;
    if (MV) {                                  // repaired blocks too: their values stay quantized
#pragma unroll
      for (int r = 0; r < NV; ++r) nvv = fmaf(p[r], wvv[r], nvv);
    }
    // meter terms p (e^c - 1).  When every bound of the wave's page is below
    // 1/4 (the common case): a short series, no exp.  Otherwise
    // 2^(l2 - m + c log2 e) - p, one exp per token, where a bound large
    // enough to overflow saturates the meter at +inf; a bound in (0, 2^-6)
    // would lose relative precision to that subtraction, so then the page
    // takes the series path with the exp for the larger bounds (both choices
    // wave-uniform).
    float ea = 0.0f, eb = 0.0f;
    if (meterA && !exact) {
      // (as unsigned bits: the bounds are >= 0, and a NaN compares above 1/4)
      uint32_t cbig = 0u;
#pragma unroll
      for (int r = 0; r < NV; ++r) cbig = max(cbig, max(__float_as_uint(cA[r]), __float_as_uint(cB[r])));
      // (the sums start from the first token's term: a 0.0f start value
      // would cost an add, since 0 + (-0) is not -0)
      float ta[NV], tb[NV];
      if (__builtin_amdgcn_ballot_w64(cbig >= 0x3E800000u) == 0) {
#pragma unroll
        for (int r = 0; r < NV; ++r) {
          ta[r] = p_expm1_small(p[r], cA[r]);
          tb[r] = meterB ? p_expm1_small(p[r], cB[r]) : 0.0f;
        }
      } else {
        // some bound in (0, 2^-6)?  As unsigned bits, c - 1 < 2^-6 - 1 exactly then
        uint32_t cmin = 0xFFFFFFFFu;
#pragma unroll
        for (int r = 0; r < NV; ++r)
          cmin = min(cmin, min(__float_as_uint(cA[r]) - 1u, __float_as_uint(cB[r]) - 1u));
        const bool tiny = cmin < 0x3C7FFFFFu;
        if (__builtin_amdgcn_ballot_w64(tiny) == 0) {
#pragma unroll
          for (int r = 0; r < NV; ++r) {
            ta[r] = __builtin_amdgcn_exp2f(fmaf(cA[r], kLog2e, dl[r])) - p[r];
            tb[r] = meterB ? __builtin_amdgcn_exp2f(fmaf(cB[r], kLog2e, dl[r])) - p[r] : 0.0f;
          }
        } else {
#pragma unroll
          for (int r = 0; r < NV; ++r) {
            ta[r] = fmaxf(p[r] * expm1_fast(cA[r]), cA[r] >= 88.0f ? INFINITY : 0.0f);
            tb[r] = meterB ? fmaxf(p[r] * expm1_fast(cB[r]), cB[r] >= 88.0f ? INFINITY : 0.0f) : 0.0f;
          }
        }
      }
      ea = ta[0];
      eb = tb[0];
#pragma unroll
      for (int r = 1; r < NV; ++r) {
        ea += ta[r];
        eb += tb[r];
      }
      na += ea;
      nb += eb;
#pragma unroll
      for (int r = 0; r < NV; ++r) {
        ca_max = vmax(ca_max, cA[r]);
        cb_max = vmax(cb_max, cB[r]);
      }
    }
    if (risk) {
      // block risks go through a per-wave LDS tile [head][16 pages] and out
      // as 16-page runs of each head's row
      if (riskmax) {                           // the tanh gate's input: the block's largest c
        float cm = 0.0f;
#pragma unroll
        for (int r = 0; r < NV; ++r) cm = vmax(cm, meterB ? cB[r] : cA[r]);
        if (CMP) cm = vmax(cm, dpp_ror8(cm));
        cm = max4k(cm);
        if (kq == 0 && n < G) sR[n][i & 15] = cm;
      } else {
        // (every lane writes: the four k lanes of head n hold the same sum,
        // and rows n >= G of the tile are never read; the terms are >= 0, so
        // a riskless block gets log 0 = -inf)
        float er = meterB ? eb : ea;
        if (CMP) er += dpp_ror8(er);
        er = sum4k(er);
        sR[n][i & 15] = (__builtin_amdgcn_logf(er) + m_ref) * kLn2;
      }
    }

    // ---------------- PV: O^T += Vhat^T P^T
    h4 Bc;
    uint4 Bp;
    uint32_t ph0 = 0, ph1 = 0, pl0 = 0, pl1 = 0;   // 16-bit store: bf16 pairs of P_hi, P_lo
    if (SCHEME == WC_BF16_STORE) {
      // p = hi + lo with hi the truncated bf16 of p and lo the bf16 of the rest
      auto split2 = [&](float x0, float x1, uint32_t& hi, uint32_t& lo) {
        const uint32_t u0 = __float_as_uint(x0) & 0xFFFF0000u, u1 = __float_as_uint(x1) & 0xFFFF0000u;
        hi = (u0 >> 16) | u1;
        lo = (__float_as_uint(x0 - __uint_as_float(u0)) >> 16) |
             (__float_as_uint(x1 - __uint_as_float(u1)) & 0xFFFF0000u);
      };
      split2(p[0], p[1], ph0, pl0);
      if (CMP) {                               // tokens 2, 3 come back from lane n + 8
        ph1 = dpp_shl8_lo(ph0, ph0);
        pl1 = dpp_shl8_lo(pl0, pl0);
      } else {
        split2(p[2], p[3], ph1, pl1);
      }
    } else if (CMP) {                          // tokens 2, 3 come back from lane n + 8
      const h2 own = {(_Float16)(p[0] * sv[0]), (_Float16)(p[1] * sv[1])};
      const uint32_t up = dpp_shl8_lo(as_u32(own), as_u32(own));
      Bc = make_h4(as_u32(own), up);
    } else {
      Bc = h4{(_Float16)(p[0] * sv[0]), (_Float16)(p[1] * sv[1]), (_Float16)(p[2] * sv[2]), (_Float16)(p[3] * sv[3])};
    }
    const uint32_t vw[8] = {vl.v0.x, vl.v0.y, vl.v0.z, vl.v0.w, vl.v1.x, vl.v1.y, vl.v1.z, vl.v1.w};
    if (SCHEME == WC_DITHER_INT8) {
      // Vhat = s (code - hb 2^-8 - lb 2^-16 + 1/2): one 16x16x32 MFMA per
      // channel tile takes the four codes and the four exact -(4 + hb 2^-8) of
      // the lane's tokens (the key side's LDS tile as it stands) against P^T
      // twice over; the 4 + 1/2 and the low byte, through its mean 255/2 (its
      // spread moves an output by < 2^-9 of one code step), are added once
      // after the loop from the sum of the weights.
      const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
      vsum = __builtin_amdgcn_fdot2(make_h2(Bc[0], Bc[1]), ones, vsum, false);
      vsum = __builtin_amdgcn_fdot2(make_h2(Bc[2], Bc[3]), ones, vsum, false);
      const h8 B2 = make_h8(as_u32(make_h2(Bc[0], Bc[1])), as_u32(make_h2(Bc[2], Bc[3])),
                            as_u32(make_h2(Bc[0], Bc[1])), as_u32(make_h2(Bc[2], Bc[3])));
      // (with the outlier bypass the address is formed here from a laundered
      // lane index, so that it holds no register through the rest of the
      // page: those instances are the ones at the register limit)
      int ln = lane;
      if (NO4 > 0) asm volatile("" : "+v"(ln));
      const uint8_t* hrow = reinterpret_cast<const uint8_t*>(sH[4 * (ln >> 4) + ((ln >> 2) & 3)]) + 64 * (ln & 3);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint32_t c0, c1;
        codes_to_h(vw[t], c0, c1);
        const uint2 hb = tr16_read(hrow + 8 * t);
        O[t] = mfma32(make_h8(c0, c1, hb.x, hb.y), B2, O[t]);
      }
    } else if (SCHEME == WC_BF16_STORE) {
      // [V|V] . [P_hi|P_lo]: tokens 4k..4k+3 of channel 8n + t twice, against
      // the bf16 attention weights and their bf16 remainders
      const uint4 vx[4] = {vl.v0, vl.v1, vl.v2, vl.v3};
      Bp = make_uint4(ph0, ph1, pl0, pl1);
      // past the end of the last page the store holds whatever was there:
      // its values are masked to 0 (their weights are 0, a NaN would not be)
      uint32_t mk0 = 0xFFFFFFFFu, mk1 = 0xFFFFFFFFu;
      if (!full) {
        const int t0 = tok0 + 4 * kq;
        mk0 = (t0 < S ? 0x0000FFFFu : 0u) | (t0 + 1 < S ? 0xFFFF0000u : 0u);
        mk1 = (t0 + 2 < S ? 0x0000FFFFu : 0u) | (t0 + 3 < S ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint4 w = vx[t >> 1];
        const uint32_t a0 = ((t & 1) ? w.z : w.x) & mk0, a1 = ((t & 1) ? w.w : w.y) & mk1;
        O[t] = mfma_bf(make_uint4(a0, a1, a0, a1), Bp, O[t]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint32_t c0, c1;
        if (SCHEME == WC_RTN_INT8)
          codes_to_h(vw[t], c0, c1);
        else
          fp8_to_h(vw[t], c0, c1);
        O[t] = mfma16(make_h4(c0, c1), Bc, O[t]);
      }
    }
    if (risk && ((i & 15) == 15 || i == npw - 1)) {
      __builtin_amdgcn_wave_barrier();
      // the lane index is laundered so that no per-lane address of this rare
      // flush is hoisted out of the loop (it would hold registers throughout)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int i0 = i & ~15, cnt = (i & 15) + 1, pj = ln & 15;
      float* rrow = a.block_logrisk + ((int64_t)b * a.Hq + g * G) * a.max_pages + w0 + i0;
      for (int q4 = 0; q4 < G; q4 += 4) {
        const int hn = (ln >> 4) + q4;
        if (hn < G && pj < cnt) rrow[(int64_t)hn * a.max_pages + pj] = sR[hn][pj];
      }
      __builtin_amdgcn_wave_barrier();
    }
  };
  if constexpr (kDepth == 1) {
    for (int i = 0; i < npw; i += 2) {
      page(kA, vA, kB, vB, i);
      if (i + 1 >= npw) break;
      page(kB, vB, kA, vA, i + 1);
    }
  } else {
    // a ring of kDepth + 1 page buffers: page i is processed while pages
    // i + 1 .. i + kDepth are in flight
    KLoad kb[kDepth + 1];
    VLoad vb[kDepth + 1];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (npw > 0) fetch(min(d, npw - 1), kb[d], vb[d]);
    for (int i = 0; i < npw; i += kDepth + 1) {
#pragma unroll
      for (int u = 0; u <= kDepth; ++u) {
        if (i + u >= npw) break;
        page(kb[u], vb[u], kb[(u + kDepth) % (kDepth + 1)], vb[(u + kDepth) % (kDepth + 1)], i + u);
      }
    }
  }
  const float m_run = m_ref;
  if (SCHEME == WC_DITHER_INT8) {                // 4 + 1/2 - (255/2) 2^-16 per unit of weight
    const float vb = sum4k(vsum) * 4.49805450439453125f;
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] += vb;
  }

  // ---------------------------------------------------------------- combine waves
  if (CMP) {
    l_run += dpp_ror8(l_run);
    na += dpp_ror8(na);
    nb += dpp_ror8(nb);
    if (MV) nvv += dpp_ror8(nvv);
    ca_max = vmax(ca_max, dpp_ror8(ca_max));
    cb_max = vmax(cb_max, dpp_ror8(cb_max));
  }
  l_run = sum4k(l_run);
  na = sum4k(na);
  nb = sum4k(nb);
  if (MV) nvv = sum4k(nvv);
  ca_max = max4k(ca_max);
  cb_max = max4k(cb_max);
  __syncthreads();                             // the dither tiles are reused below
  float (*sO)[16][128] = reinterpret_cast<float (*)[16][128]>(smem);
  __shared__ float sM[kNW][16][7];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r)                // row 4k + r of tile t: channel 32k + 4t + r (16-bit store: 32k + 8r + t)
      sO[wave][n][SCHEME == WC_BF16_STORE ? 32 * kq + 8 * r + t : 32 * kq + 4 * t + r] = O[t][r];
  if (kq == 0) {
    sM[wave][n][0] = m_run;
    sM[wave][n][1] = l_run;
    sM[wave][n][2] = na;
    sM[wave][n][3] = nb;
    sM[wave][n][4] = ca_max;
    sM[wave][n][5] = cb_max;
    sM[wave][n][6] = nvv;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * kPartial; e += kThreads) {
    const int hn = e / kPartial, f = e % kPartial;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, sM[w][hn][0]);
    float val = 0.0f;
    if (f == 0) {
      val = M;
    } else if (f >= 132 && f != 134) {         // largest bounds: max over the waves
      if (f < 134) {
#pragma unroll
        for (int w = 0; w < kNW; ++w) val = fmaxf(val, sM[w][hn][f - 128]);
      }
    } else if (f == 134) {                     // value certificate sum, rescaled like l
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
          const float mw = sM[w][hn][0];
          val = fmaf(mw == -INFINITY ? 0.0f : exp2f(mw - M), sM[w][hn][6], val);
        }
      }
    } else if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float mw = sM[w][hn][0];
        const float sc = mw == -INFINITY ? 0.0f : exp2f(mw - M);
        const float x = f < 4 ? sM[w][hn][f] : sO[w][hn][f - 4];
        val = fmaf(sc, x, val);
      }
    }
    a.partials[(((int64_t)b * a.Hq + g * G + hn) * a.n_split + split) * kPartial + f] = val;
  }
}

// ---------------------------------------------------------------- LSE merge
// One wave per (b, h).  Lanes take the splits for the maxima and the scalar
// sums (wave reductions), then two output channels each with the split loop
// unrolled so that its loads are in flight together.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += shfl_xor(v, m);
  return v;
}

// ---------------------------------------------------------------- load floor
// What HBM delivers for the decode's own access pattern: the same grid, page
// assignment, page-table batches, buffer resources, cache policies and page
// loads as decode_kernel (kDepth = 1: one page in flight ahead of the one in
// hand), with no arithmetic.  Each lane folds every loaded word into one
// xor, stored only if it equals a fixed pattern, so that no load is dropped.
// Dynamic LDS (the decode instance's static size) gives it the decode's
// residency per CU.  The query, the outlier side store and the value
// witnesses are not read.
struct FloorArgs {
  const int32_t* page_table;
  const int32_t* ctx_len;
  uint32_t* sink;
  int max_pages, n_split, layer, meterA;
};

__device__ __forceinline__ uint32_t fold4(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }
__device__ __forceinline__ uint32_t fold4(float4 v) { return fold4(__builtin_bit_cast(uint4, v)); }

template <int SCHEME, bool PAIR>
__global__ void __launch_bounds__(kThreads) decode_floor_kernel(wc_cache c, FloorArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int S = a.ctx_len[b];
  const int P = (S + 15) >> 4;
  const int p0 = (int)((int64_t)split * P / a.n_split), p1 = (int)((int64_t)(split + 1) * P / a.n_split);
  const bool meterA = a.meterA != 0;
  const int r0 = PAIR ? 2 * (n >> 3) : 0;
  LaneOff lo;
  lo.k = (uint32_t)(16 * lane);
  lo.s = (uint32_t)(4 * (4 * kq + r0));
  lo.w = meterA ? (uint32_t)(4 * (8 * n + 2 * kq)) : lo.k;
  lo.v = (uint32_t)(16 * lane);
  lo.o = 0;
  const int per = (p1 - p0 + kNW - 1) / kNW;
  const int w0 = p0 + wave * per;
  const int npw = max(0, min(p1, w0 + per) - w0);
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
  const int64_t pg_base = (int64_t)a.layer * c.num_pages;
  const int64_t lph = c.num_pages * c.num_kv_heads;
  const int64_t l0 = (int64_t)a.layer * lph;
  constexpr int64_t PB = page_bytes<SCHEME>();
  LayerBufs lb;
  lb.k = layer_rsrc(c.k_codes, l0 * PB, (uint64_t)lph * PB);
  lb.v = layer_rsrc(c.v_codes, l0 * PB, (uint64_t)lph * PB);
  lb.w = meterA ? layer_rsrc(c.witness, l0 * 512, (uint64_t)lph * 512) : lb.k;
  lb.o = lb.ks = lb.vs = lb.wv = lb.k;
  if (int8_codes<SCHEME>()) {
    lb.ks = layer_rsrc(c.k_scale, l0 * 64, (uint64_t)lph * 64);
    lb.vs = layer_rsrc(c.v_scale, l0 * 64, (uint64_t)lph * 64);
  }
  uint32_t acc = 0;
  int bphys = 0, bslot = -1;
  auto fetch = [&](int i, KLoad& d, VLoad& e) {
    if (i >= npw) {                            // past the last page: physical page 0, as the decode
      d.slot = -1;
      load_page_soff<SCHEME, PAIR, 0, false>(lb, (uint32_t)g, lo, meterA, d, e);
      return;
    }
    if ((i & 63) == 0) {
      const int j = i + lane;
      const int ph = j < npw ? ptab[w0 + j] : 0;
      const int sl = (j < npw && c.exact_slot) ? c.exact_slot[(pg_base + ph) * c.num_kv_heads + g] : -1;
      bphys = settle(ph);
      bslot = settle(sl);
    }
    const int phys = __builtin_amdgcn_readlane(bphys, i & 63);
    d.slot = __builtin_amdgcn_readlane(bslot, i & 63);
    load_page_soff<SCHEME, PAIR, 0, false>(lb, (uint32_t)(phys * c.num_kv_heads + g), lo, meterA, d, e);
  };
  auto fold = [&](const KLoad& d, const VLoad& e) {
    uint32_t x = fold4(d.k0) ^ fold4(d.k1) ^ fold4(e.v0) ^ fold4(e.v1) ^ (uint32_t)d.slot;
    if (SCHEME == WC_BF16_STORE) x ^= fold4(d.k2) ^ fold4(d.k3) ^ fold4(e.v2) ^ fold4(e.v3);
    if (meterA) x ^= __float_as_uint(d.w.x) ^ __float_as_uint(d.w.y);
    if (int8_codes<SCHEME>()) x ^= fold4(d.ks) ^ fold4(e.vs);
    acc = (acc << 1 | acc >> 31) ^ x;
  };
  KLoad kA, kB;
  VLoad vA, vB;
  if (npw > 0) fetch(0, kA, vA);
  for (int i = 0; i < npw; i += 2) {
    fetch(i + 1, kB, vB);
    fold(kA, vA);
    if (i + 1 >= npw) break;
    fetch(i + 2, kA, vA);
    fold(kB, vB);
  }
  if (acc == 0x9E3779B9u) a.sink[0] = acc;
}

__global__ void __launch_bounds__(64) merge_kernel(const float* __restrict__ part, int n_split, float* o,
                                                   float* lse, float* meter_a, float* meter_b, float* tanh_a,
                                                   float* tanh_b, float* meter_v) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const float* pp = part + (int64_t)bh * n_split * kPartial;
  float M = -INFINITY;
  for (int s = lane; s < n_split; s += 64) M = fmaxf(M, pp[s * kPartial]);
  M = wave_max(M);
  auto weight = [&](float ms) { return (ms == -INFINITY || M == -INFINITY) ? 0.0f : exp2f(ms - M); };
  float L = 0.f, NA = 0.f, NB = 0.f, CA = 0.f, CB = 0.f, NV = 0.f;
  for (int s = lane; s < n_split; s += 64) {
    const float4 q = *reinterpret_cast<const float4*>(pp + s * kPartial);
    const float4 cm = *reinterpret_cast<const float4*>(pp + s * kPartial + 132);
    const float w = weight(q.x);
    L = fmaf(w, q.y, L);
    NA = fmaf(w, q.z, NA);
    NB = fmaf(w, q.w, NB);
    CA = fmaxf(CA, cm.x);
    CB = fmaxf(CB, cm.y);
    NV = fmaf(w, cm.z, NV);
  }
  L = wave_sum(L);
  NA = wave_sum(NA);
  NB = wave_sum(NB);
  NV = wave_sum(NV);
  CA = wave_max(CA);
  CB = wave_max(CB);
  float o0 = 0.f, o1 = 0.f;
  int s = 0;
  for (; s + 8 <= n_split; s += 8) {
    float mw[8];
    float2 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      mw[k] = pp[(s + k) * kPartial];
      v[k] = *reinterpret_cast<const float2*>(pp + (s + k) * kPartial + 4 + 2 * lane);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = weight(mw[k]);
      o0 = fmaf(w, v[k].x, o0);
      o1 = fmaf(w, v[k].y, o1);
    }
  }
  for (; s < n_split; ++s) {
    const float w = weight(pp[s * kPartial]);
    const float2 v = *reinterpret_cast<const float2*>(pp + s * kPartial + 4 + 2 * lane);
    o0 = fmaf(w, v.x, o0);
    o1 = fmaf(w, v.y, o1);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float2*>(o + (int64_t)bh * 128 + 2 * lane) = make_float2(o0 * inv, o1 * inv);
  if (lane == 0) {
    lse[bh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
    const float ea = NA * inv, eb = NB * inv;
    if (meter_a) meter_a[bh] = ea * (1.0f + 0.5f * ea);
    if (meter_b) meter_b[bh] = eb * (1.0f + 0.5f * eb);
    if (tanh_a) tanh_a[bh] = tanhf(0.5f * CA);
    if (tanh_b) tanh_b[bh] = tanhf(0.5f * CB);
    if (meter_v) meter_v[bh] = NV * inv;
  }
}

// The merge for at most 16 splits in one round of loads: lane s < n_split
// reads split s's scalars, every lane reads its two output channels of
// every split, all before the first wait; the maxima and sums over the
// splits are DPP reductions within the first 16 lanes.
__global__ void __launch_bounds__(64) merge16_kernel(const float* __restrict__ part, int n_split, float* o,
                                                     float* lse, float* meter_a, float* meter_b, float* tanh_a,
                                                     float* tanh_b, float* meter_v) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const float* pp = part + (int64_t)bh * n_split * kPartial;
  float2 v[16];
#pragma unroll
  for (int s = 0; s < 16; ++s)
    v[s] = s < n_split ? *reinterpret_cast<const float2*>(pp + s * kPartial + 4 + 2 * lane) : make_float2(0.f, 0.f);
  const bool mine = lane < n_split;
  const float4 q = mine ? *reinterpret_cast<const float4*>(pp + lane * kPartial) : make_float4(-INFINITY, 0.f, 0.f, 0.f);
  const float4 cm = mine ? *reinterpret_cast<const float4*>(pp + lane * kPartial + 132) : make_float4(0.f, 0.f, 0.f, 0.f);
  // lanes 16 .. 63 hold -inf and zeros: the row-0 reductions are the totals
  const float M = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_max(q.x))));
  const float w = (q.x == -INFINITY || M == -INFINITY) ? 0.0f : exp2f(q.x - M);
  const float L = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_sum(w * q.y))));
  const float NA = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_sum(w * q.z))));
  const float NB = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_sum(w * q.w))));
  const float NV = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_sum(w * cm.z))));
  const float CA = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_max(cm.x))));
  const float CB = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row16_max(cm.y))));
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s < n_split) {
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
      o0 = fmaf(ws, v[s].x, o0);
      o1 = fmaf(ws, v[s].y, o1);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float2*>(o + (int64_t)bh * 128 + 2 * lane) = make_float2(o0 * inv, o1 * inv);
  if (lane == 0) {
    lse[bh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
    const float ea = NA * inv, eb = NB * inv;
    if (meter_a) meter_a[bh] = ea * (1.0f + 0.5f * ea);
    if (meter_b) meter_b[bh] = eb * (1.0f + 0.5f * eb);
    if (tanh_a) tanh_a[bh] = tanhf(0.5f * CA);
    if (tanh_b) tanh_b[bh] = tanhf(0.5f * CB);
    if (meter_v) meter_v[bh] = NV * inv;
  }
}

}  // namespace wc

using namespace wc;

extern "C" size_t wc_decode_workspace_bytes(int B, int Hq, int n_split) {
  if (B < 0 || Hq < 0 || n_split < 0) return 0;
  return (size_t)B * Hq * n_split * kPartial * sizeof(float);
}

// Host dispatch from the run-time shape to the template instance.  The meter
// configurations of the common shapes (bf16 query, group <= 8, 32-bit layer
// offsets, no value certificate; with or without the outlier bypass) have
// instances of their own.
template <int SCH, bool QF, bool CM, bool SO, int NO>
static void launch_mv(bool mv, int mode, dim3 grid, hipStream_t st, const wc_cache& c, const DecodeArgs& a) {
  if constexpr (!QF && CM && SO) {
    if (!mv && mode == kModeOff) {
      hipLaunchKernelGGL((decode_kernel<SCH, QF, CM, SO, NO, false, kModeOff>), grid, dim3(kThreads), 0, st, c, a);
      return;
    }
    if (!mv && mode == kModeOn) {
      hipLaunchKernelGGL((decode_kernel<SCH, QF, CM, SO, NO, false, kModeOn>), grid, dim3(kThreads), 0, st, c, a);
      return;
    }
  }
  if (mv)
    hipLaunchKernelGGL((decode_kernel<SCH, QF, CM, SO, NO, true, kModeRuntime>), grid, dim3(kThreads), 0, st, c, a);
  else
    hipLaunchKernelGGL((decode_kernel<SCH, QF, CM, SO, NO, false, kModeRuntime>), grid, dim3(kThreads), 0, st, c, a);
}
template <int SCH, bool QF, bool CM, bool SO>
static void launch_no(int no4, bool mv, int mode, dim3 grid, hipStream_t st, const wc_cache& c, const DecodeArgs& a) {
  if constexpr (SCH == WC_DITHER_INT8) {
    if (no4 == 2) return launch_mv<SCH, QF, CM, SO, 2>(mv, mode, grid, st, c, a);
    if (no4 == 4) return launch_mv<SCH, QF, CM, SO, 4>(mv, mode, grid, st, c, a);
  }
  launch_mv<SCH, QF, CM, SO, 0>(mv, mode, grid, st, c, a);
}
template <int SCH, bool QF>
static void launch_shape(bool cm, bool so, int no4, bool mv, int mode, dim3 grid, hipStream_t st, const wc_cache& c,
                         const DecodeArgs& a) {
  if (cm) {
    if (so) launch_no<SCH, QF, true, true>(no4, mv, mode, grid, st, c, a);
    else launch_no<SCH, QF, true, false>(no4, mv, mode, grid, st, c, a);
  } else {
    if (so) launch_no<SCH, QF, false, true>(no4, mv, mode, grid, st, c, a);
    else launch_no<SCH, QF, false, false>(no4, mv, mode, grid, st, c, a);
  }
}
template <bool QF>
static void launch_scheme(int scheme, bool cm, bool so, int no4, bool mv, int mode, dim3 grid, hipStream_t st,
                          const wc_cache& c, const DecodeArgs& a) {
  switch (scheme) {
    case WC_DITHER_INT8: launch_shape<WC_DITHER_INT8, QF>(cm, so, no4, mv, mode, grid, st, c, a); break;
    case WC_FP8_E4M3: launch_shape<WC_FP8_E4M3, QF>(cm, so, no4, mv, mode, grid, st, c, a); break;
    case WC_RTN_INT8: launch_shape<WC_RTN_INT8, QF>(cm, so, no4, mv, mode, grid, st, c, a); break;
    default: launch_shape<WC_BF16_STORE, QF>(cm, so, no4, mv, mode, grid, st, c, a); break;
  }
}

extern "C" int wc_decode_attn_meter(const wc_cache* cache, int layer, const void* q, int q_dtype, int B, int Hq,
                                    const int32_t* page_table, int max_pages, const int32_t* ctx_len,
                                    const uint64_t* seed, float sm_scale, unsigned meter_mask, double delta_req,
                                    int L, int H, int T, int n_split, float* partials, size_t ws_bytes,
                                    float* block_logrisk, void* stream) {
  if (!cache || (B != 0 && (!q || !page_table || !ctx_len || !partials))) {
    set_error("wc_decode_attn_meter: null pointer");
    return WC_EINVAL;
  }
  const wc_cache& c = *cache;
  if (c.head_dim != 128 || c.num_bands != 8 || c.page_size != 16 || c.num_kv_heads < 1 || c.num_pages < 1) {
    // (a wave's prefetch past its last page, or of a wave with no page,
    // requests physical page 0, so the layer needs one)
    set_error("wc_decode_attn_meter: need head_dim 128, 8 bands, 16-token pages, >= 1 physical page");
    return WC_EUNSUPPORTED;
  }
  if (c.scheme != WC_DITHER_INT8 && c.scheme != WC_FP8_E4M3 && c.scheme != WC_RTN_INT8 &&
      c.scheme != WC_BF16_STORE) {
    set_error("wc_decode_attn_meter: scheme %d has no decode path", c.scheme);
    return WC_EUNSUPPORTED;
  }
  if (q_dtype != WC_F32 && q_dtype != WC_BF16) {
    set_error("wc_decode_attn_meter: q_dtype must be WC_F32 or WC_BF16");
    return WC_EUNSUPPORTED;
  }
  if (B < 0 || Hq < 1 || Hq % c.num_kv_heads != 0 || Hq / c.num_kv_heads > 16 || max_pages < 1 ||
      n_split < 1 || n_split > 1024 || layer < 0 || layer >= c.num_layers) {
    set_error("wc_decode_attn_meter: bad B/Hq/max_pages/n_split/layer");
    return WC_EINVAL;
  }
  if (meter_mask & ~(WC_METER_A | WC_METER_B | WC_BLOCK_CMAX | WC_METER_V)) {
    set_error("wc_decode_attn_meter: unknown meter_mask bits");
    return WC_EINVAL;
  }
  if ((meter_mask & WC_METER_B) && (c.scheme != WC_DITHER_INT8 || !(meter_mask & WC_METER_A))) {
    set_error("wc_decode_attn_meter: Tier B needs the dithered INT8 scheme and Tier A");
    return WC_EINVAL;
  }
  if ((meter_mask & WC_METER_A) && !c.witness) {
    set_error("wc_decode_attn_meter: Tier A needs the witness");
    return WC_EINVAL;
  }
  if (block_logrisk && !(meter_mask & WC_METER_A)) {
    set_error("wc_decode_attn_meter: block risks need the meter on");
    return WC_EINVAL;
  }
  if ((meter_mask & WC_METER_V) && !c.v_witness) {
    set_error("wc_decode_attn_meter: the value certificate needs the value witness");
    return WC_EINVAL;
  }
  if ((meter_mask & WC_BLOCK_CMAX) && !block_logrisk) {
    set_error("wc_decode_attn_meter: WC_BLOCK_CMAX needs the block output");
    return WC_EINVAL;
  }
  if (c.scheme == WC_DITHER_INT8 && ((!seed && B != 0) || !c.k_scale || !c.v_scale)) {
    set_error("wc_decode_attn_meter: INT8 cache needs seeds and scales");
    return WC_EINVAL;
  }
  if (c.scheme == WC_RTN_INT8 && (!c.k_scale || !c.v_scale)) {
    set_error("wc_decode_attn_meter: RTN INT8 cache needs scales");
    return WC_EINVAL;
  }
  if (!c.k_codes || !c.v_codes) {
    set_error("wc_decode_attn_meter: cache codes not set");
    return WC_EINVAL;
  }
  if (c.exact_slot && !c.exact_pool) {
    set_error("wc_decode_attn_meter: exact_slot set without exact_pool");
    return WC_EINVAL;
  }
  if (c.num_outliers != 0) {
    if (c.scheme != WC_DITHER_INT8 || (c.num_outliers != 8 && c.num_outliers != 16)) {
      set_error("wc_decode_attn_meter: the outlier bypass needs the dithered INT8 scheme and m = 8 or 16");
      return WC_EUNSUPPORTED;
    }
    if (!c.outlier_ch || !c.k_outlier) {
      set_error("wc_decode_attn_meter: outlier bypass needs outlier_ch and k_outlier");
      return WC_EINVAL;
    }
  }
  if (!(sm_scale > 0.0f) || !(delta_req > 0.0 && delta_req < 1.0) || L < 1 || H < 1 || T < 1) {
    set_error("wc_decode_attn_meter: need sm_scale > 0, 0 < delta_req < 1, L, H, T >= 1");
    return WC_EINVAL;
  }
  if (ws_bytes < wc_decode_workspace_bytes(B, Hq, n_split)) {
    set_error("wc_decode_attn_meter: workspace %zu < %zu bytes", ws_bytes, wc_decode_workspace_bytes(B, Hq, n_split));
    return WC_EWORKSPACE;
  }
  if (B == 0) return WC_OK;
  const double dloc = delta_req / ((double)L * (double)H * (double)T);
  DecodeArgs a{q, page_table, ctx_len, seed, partials, block_logrisk, B, Hq, Hq / c.num_kv_heads, max_pages,
               n_split, layer, meter_mask, sm_scale, (float)(-log(dloc))};
  dim3 grid((unsigned)n_split, (unsigned)c.num_kv_heads, (unsigned)B);
  hipStream_t st = (hipStream_t)stream;
  const bool cmp = a.G <= 8;
  // one buffer resource per layer array when its byte offsets fit 32 bits
  const uint64_t page_b = c.scheme == WC_BF16_STORE ? 4096u : 2048u;
  const bool soff = (uint64_t)c.num_pages * (uint64_t)c.num_kv_heads * page_b <= 0xFFFFFFFFull;
  const int no4 = c.scheme == WC_DITHER_INT8 ? c.num_outliers / 4 : 0;
  const bool mv = (meter_mask & WC_METER_V) != 0;
  // the fixed meter configurations: off; on (Tier A, and B for dithered INT8)
  const unsigned full = c.scheme == WC_DITHER_INT8 ? (WC_METER_A | WC_METER_B) : WC_METER_A;
  int mode = kModeRuntime;
  if (meter_mask == 0) mode = kModeOff;
  else if (meter_mask == full) mode = kModeOn;
  if (q_dtype == WC_BF16)
    launch_scheme<false>(c.scheme, cmp, soff, no4, mv, mode, grid, st, c, a);
  else
    launch_scheme<true>(c.scheme, cmp, soff, no4, mv, mode, grid, st, c, a);
  return check_launch("wc_decode_attn_meter");
}

template <int SCHEME>
static void launch_floor(bool pair, bool match, dim3 grid, hipStream_t st, const wc_cache& c, const FloorArgs& a) {
  // the residency of the decode's instance for the same cache and query
  // group (meter on, bf16 query): its static LDS, given here as dynamic LDS
  size_t lds = 0;
  if (match) {
    hipFuncAttributes fa{};
    const void* fn = pair ? reinterpret_cast<const void*>(&decode_kernel<SCHEME, false, true, true, 0, false, kModeOn>)
                          : reinterpret_cast<const void*>(&decode_kernel<SCHEME, false, false, true, 0, false, kModeOn>);
    if (hipFuncGetAttributes(&fa, fn) == hipSuccess) lds = fa.sharedSizeBytes;
  }
  if (pair)
    hipLaunchKernelGGL((decode_floor_kernel<SCHEME, true>), grid, dim3(kThreads), lds, st, c, a);
  else
    hipLaunchKernelGGL((decode_floor_kernel<SCHEME, false>), grid, dim3(kThreads), lds, st, c, a);
}

extern "C" int wc_decode_load_floor(const wc_cache* cache, int layer, int B, int Hq, const int32_t* page_table,
                                    int max_pages, const int32_t* ctx_len, int n_split, unsigned meter_mask,
                                    int match_residency, uint32_t* sink, void* stream) {
  if (!cache || (B != 0 && (!page_table || !ctx_len || !sink))) {
    set_error("wc_decode_load_floor: null pointer");
    return WC_EINVAL;
  }
  const wc_cache& c = *cache;
  if (c.head_dim != 128 || c.num_bands != 8 || c.page_size != 16 || c.num_kv_heads < 1 || c.num_pages < 1) {
    // (a wave's prefetch past its last page, or of a wave with no page,
    // requests physical page 0, so the layer needs one)
    set_error("wc_decode_load_floor: need head_dim 128, 8 bands, 16-token pages, >= 1 physical page");
    return WC_EUNSUPPORTED;
  }
  if (c.scheme != WC_DITHER_INT8 && c.scheme != WC_FP8_E4M3 && c.scheme != WC_RTN_INT8 &&
      c.scheme != WC_BF16_STORE) {
    set_error("wc_decode_load_floor: scheme %d has no decode path", c.scheme);
    return WC_EUNSUPPORTED;
  }
  if (B < 0 || Hq < 1 || Hq % c.num_kv_heads != 0 || Hq / c.num_kv_heads > 16 || max_pages < 1 ||
      n_split < 1 || n_split > 1024 || layer < 0 || layer >= c.num_layers) {
    set_error("wc_decode_load_floor: bad B/Hq/max_pages/n_split/layer");
    return WC_EINVAL;
  }
  if (meter_mask & ~(WC_METER_A | WC_METER_B | WC_BLOCK_CMAX | WC_METER_V)) {
    set_error("wc_decode_load_floor: unknown meter_mask bits");
    return WC_EINVAL;
  }
  if ((meter_mask & WC_METER_A) && !c.witness) {
    set_error("wc_decode_load_floor: Tier A needs the witness");
    return WC_EINVAL;
  }
  if ((c.scheme == WC_DITHER_INT8 || c.scheme == WC_RTN_INT8) && (!c.k_scale || !c.v_scale)) {
    set_error("wc_decode_load_floor: INT8 cache needs scales");
    return WC_EINVAL;
  }
  if (!c.k_codes || !c.v_codes) {
    set_error("wc_decode_load_floor: cache codes not set");
    return WC_EINVAL;
  }
  const uint64_t page_b = c.scheme == WC_BF16_STORE ? 4096u : 2048u;
  if ((uint64_t)c.num_pages * (uint64_t)c.num_kv_heads * page_b > 0xFFFFFFFFull) {
    set_error("wc_decode_load_floor: a layer's code array must be under 4 GB");
    return WC_EUNSUPPORTED;
  }
  if (B == 0) return WC_OK;
  FloorArgs a{page_table, ctx_len, sink, max_pages, n_split, layer, (meter_mask & WC_METER_A) ? 1 : 0};
  dim3 grid((unsigned)n_split, (unsigned)c.num_kv_heads, (unsigned)B);
  hipStream_t st = (hipStream_t)stream;
  const bool pair = Hq / c.num_kv_heads <= 8;
  const bool match = match_residency != 0;
  switch (c.scheme) {
    case WC_DITHER_INT8: launch_floor<WC_DITHER_INT8>(pair, match, grid, st, c, a); break;
    case WC_FP8_E4M3: launch_floor<WC_FP8_E4M3>(pair, match, grid, st, c, a); break;
    case WC_RTN_INT8: launch_floor<WC_RTN_INT8>(pair, match, grid, st, c, a); break;
    default: launch_floor<WC_BF16_STORE>(pair, match, grid, st, c, a); break;
  }
  return check_launch("wc_decode_load_floor");
}

extern "C" int wc_lse_merge(const float* partials, int B, int Hq, int n_split, float* o, float* lse,
                            float* meter_a, float* meter_b, float* tanh_a, float* tanh_b, float* meter_v,
                            void* stream) {
  if ((B != 0 && (!partials || !o || !lse)) || B < 0 || Hq < 1 || n_split < 1 || n_split > 1024) {
    set_error("wc_lse_merge: bad arguments");
    return WC_EINVAL;
  }
  if (B == 0) return WC_OK;
  if (n_split <= 16)
    hipLaunchKernelGGL(merge16_kernel, dim3((unsigned)(B * Hq)), dim3(64), 0, (hipStream_t)stream, partials, n_split,
                       o, lse, meter_a, meter_b, tanh_a, tanh_b, meter_v);
  else
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(B * Hq)), dim3(64), 0, (hipStream_t)stream, partials, n_split, o,
                       lse, meter_a, meter_b, tanh_a, tanh_b, meter_v);
  return check_launch("wc_lse_merge");
}
