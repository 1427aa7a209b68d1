/*
 * witcert.h -- C ABI of the MI355X (gfx950) WitCert hot path.
 *
 * WitCert ("WitCert: Sound Runtime Risk Observability and Gating for
 * KV-Cache Quantization", arXiv 2607.28699) stores, at write time, a
 * per-band residual-norm witness beside a quantized KV cache and computes,
 * in the same pass as decode attention, a per-(layer, head, step) upper
 * bound on the total variation between exact and compressed attention.
 * The implementation paragraph of the m.montaan.com summary lists the four
 * pieces exported here: a write path storing witnesses, a fused decode
 * attention kernel computing output and meter in one data pass, LSE-merged
 * certificate accumulation across KV splits, and a gate that pages in exact
 * blocks from a CPU backing store when the meter exceeds a threshold.
 *
 * Conventions
 *  - The caller owns every buffer.  Device buffers come from any allocator
 *    (PyTorch here); the exact backing store is pinned host memory that the
 *    device can read (hipHostMalloc / torch pin_memory).  The library never
 *    allocates or frees, and keeps no state beyond a thread-local error text.
 *  - Every call is asynchronous on the HIP stream passed as `stream`
 *    (a hipStream_t; NULL = the default stream) and never synchronizes.
 *  - Shapes are validated on the host before any launch.  Return codes:
 *      WC_OK 0, WC_EINVAL -1 (null pointer, bad shape or argument),
 *      WC_EUNSUPPORTED -2 (scheme/dtype/shape not built),
 *      WC_EWORKSPACE -3 (workspace too small), WC_EHIP -4 (launch error).
 *    wc_last_error() returns a text for the last failure on this thread.
 *  - A call with nothing to do (n_tok = 0, n_pages = 0 or B = 0) checks its
 *    other arguments and returns WC_OK without a launch; its data pointers
 *    may then be NULL (the cache descriptor may not).
 *  - Device-resident index arrays (slots, positions, page tables, lengths)
 *    cannot be checked on the host: out-of-range values are undefined
 *    behaviour, as for any kernel argument.
 *
 * Cache layout (one layer = `num_pages` physical pages; arrays carry a
 * leading layer dimension of `num_layers`; P = num_pages, Hkv = num_kv_heads,
 * d = 128, page = 16 tokens for INT8/fp8, 32 for 2-bit):
 *  k_codes   INT8/fp8: [L][P][Hkv][2][4][16][16] bytes per page-head
 *            block: token t, channel c at [(c%32)/16][c/32][t][c%16] (each
 *            1 KB half holds, for every token, 16 channels of each 32-channel
 *            group).  INT8 codes (dithered and RTN) are stored as offset
 *            binary (code + 128).
 *            16-bit store: bf16 [L][P][Hkv][4][4][16][8]: token t, channel c
 *            at [(c%32)/8][c/32][t][c%8] (4 KB per page-head block).
 *            2-bit:    [L][P][Hkv][128][8] bytes (32 tokens of one channel,
 *                      4 codes per byte, token i in bits 2(i%4)).
 *  v_codes   INT8/fp8: [L][P][Hkv][2][4][16][4][4] bytes: token t, channel c
 *                      at [(c%32)/16][t/4][4(c/32) + c%4][(c%16)/4][t%4]
 *                      (four tokens of one channel are one 32-bit word).
 *            2-bit:    [L][P][Hkv][32][32] bytes (token-major, 4 codes/byte).
 *            16-bit store: bf16 [L][P][Hkv][4][4][16][2][4]: token t,
 *                      channel c at [(c%8)/2][t/4][c/8][c%2][t%4].
 *  k_scale,
 *  v_scale   INT8 (dithered and RTN): fp32 [L][P][Hkv][16], s = absmax/127
 *            of the row.
 *  k_aux     2-bit: fp32 [L][P][Hkv][128][2] (scale, min) per channel group.
 *  v_aux     2-bit: fp32 [L][P][Hkv][32][4][2] (scale, min) per token group.
 *  witness   fp32 [L][P][Hkv][page][8]: w_{t,b} = ||r_{t,b}||, keys only.
 *  exact_slot int32 [L][P][Hkv]: -1 = quantized, else the slot of the
 *            repaired block in the exact pool.  A caller that hands a
 *            physical page to another sequence resets its entries to -1.
 *  exact_pool bf16 [capacity][16][128]: a repaired block's exact keys, token
 *            t of the block at row t (row t of slot s at (16 s + t) * 128).
 *  outlier_ch int32 [L][Hkv][m] (m = num_outliers): the outlier-bypass
 *            channels O of each layer and KV head, ascending and distinct.
 *  k_outlier bf16 [L][P][Hkv][16][m]: entry i of a token is its exact key on
 *            channel O[i].
 *  v_witness fp32 [L][P][Hkv][page]: the value witness w^V_t = ||v^_t - v_t||
 *            over all 128 channels (written when the pointer is set).
 *
 * Exact keys and repair (the gate).  The exact store is bf16: the pinned host
 * store, the exact pool and the keys the write path copies into it.  A
 * repaired block's tokens are decoded with their exact keys and c_t = 0, so
 * a cache with exact_slot set takes bf16 keys only (wc_write_kv,
 * wc_write_kv_pages and the key witness of wc_witness refuse float32 keys
 * with WC_EUNSUPPORTED).  Repair persists (paperswithlean Figure 5 caption:
 * incremental persistent repair): a token written into a repaired block also
 * gets its exact key in the block's pool row and a zero witness, so appends
 * into a partially filled repaired page stay exact.  The host store must hold
 * the exact keys of every token written before a gate call that may repair
 * its block.
 *
 * Value certificate (WC_METER_V).  The summary reports joint K+V coverage but
 * defines witnesses for keys only.  Reading implemented here: the value
 * witness above, and E_V = sum_t p~_t w^V_t, which bounds the value part of
 * the output error, ||sum_t p~_t (v^_t - v_t)||, by the triangle inequality
 * for any value quantizer; with the key side's TV,
 * ||o~ - o|| <= E_V + 2 TV max_t ||v_t||.  E_V is taken on the stored v^.  For
 * dithered INT8 the returned output uses each value draw's low byte at its
 * mean (every dequantized value within 2^-9 of its code step of v^), so the
 * bound on the output this library returns adds 2^-9 sqrt(128) sum_t p~_t s_t
 * <= 2^-9 sqrt(128) max_t s_t (s_t the value row scale); other schemes add 0.
 *
 * Outlier bypass (dithered INT8 keys, m = 8 or 16).  The summary reports the
 * capacity of the certified INT8 cache with an outlier bypass too, and
 * results per outlier budget m (capacity and negative-results paragraphs);
 * the pages give no more detail.  Reading implemented here: the m channels of largest key
 * energy of a (layer, KV head) (wc_outlier_select) are stored exactly in
 * k_outlier; the row scale is the absmax of the other channels, the INT8 code
 * on O is 0 and the residual there is 0 (so is its share of the witness); the
 * decode adds the exact O part of each logit, and Tier B sums q_c^2 over the
 * channels off O only (s_{c,t} = 0 on O in the Tier B paragraph's proxy).
 * Values are not bypassed.
 */
#ifndef WITCERT_H
#define WITCERT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WC_OK 0
#define WC_EINVAL (-1)
#define WC_EUNSUPPORTED (-2)
#define WC_EWORKSPACE (-3)
#define WC_EHIP (-4)

/* Quantization schemes. */
#define WC_DITHER_INT8 0 /* subtractively-dithered INT8 (Tier A + Tier B) */
#define WC_FP8_E4M3 1    /* fp8 e4m3fn raw cast, black box (Tier A)       */
#define WC_KIVI2 2       /* 2-bit asymmetric, group 32 (write path only)  */
#define WC_RTN_INT8 3    /* round-to-nearest INT8, black box (Tier A)     */
#define WC_BF16_STORE 4  /* 16-bit store of any scheme's output x^ (Tier A,
                            witness through wc_witness)                   */

/* Input dtypes. */
#define WC_F32 0
#define WC_BF16 1

/* meter_mask bits. */
#define WC_METER_A 1u
#define WC_METER_B 2u
#define WC_BLOCK_CMAX 4u /* block output = largest per-token bound (tanh gate) */
#define WC_METER_V 8u    /* value certificate (needs cache->v_witness)       */

typedef struct {
  int32_t scheme;       /* WC_DITHER_INT8 | WC_FP8_E4M3 | WC_KIVI2          */
  int32_t head_dim;     /* must be 128                                       */
  int32_t num_kv_heads; /* Hkv >= 1                                          */
  int32_t num_bands;    /* must be 8: band b = frequency pairs [8b, 8b+8)    */
  int32_t page_size;    /* 16 (INT8, fp8) or 32 (2-bit)                      */
  int32_t num_layers;   /* leading dimension of every cache array            */
  int64_t num_pages;    /* physical pages per layer                          */
  void* k_codes;
  void* v_codes;
  float* k_scale;
  float* v_scale;
  float* k_aux;
  float* v_aux;
  float* witness;
  int32_t* exact_slot;  /* may be NULL when no block is ever repaired        */
  uint16_t* exact_pool; /* bf16 [pool_capacity][16][128]                     */
  int64_t pool_capacity;
  int32_t num_outliers; /* m: 0 (no bypass), 8 or 16 (dithered INT8 only)     */
  int32_t reserved;     /* 0                                                 */
  int32_t* outlier_ch;  /* [L][Hkv][m] when m > 0                            */
  uint16_t* k_outlier;  /* bf16 [L][P][Hkv][16][m] when m > 0                */
  float* v_witness;     /* fp32 [L][P][Hkv][page]: ||v^_t - v_t|| (nullable) */
} wc_cache;

/*
 * wc_write_kv -- quantize keys and values and store their witnesses.
 *
 * Defined by the WitCert summary: subtractive dither x^ = s(round(x/s + xi)
 * - xi) with xi regenerated at read time (Tier B paragraph), the witness
 * w_{t,b} = ||r_{t,b}|| stored once per token at write time (witness-theorem
 * paragraph), and black-box schemes measured through the same witness
 * (implementation paragraph; fp8 raw and kivi-2bit in the RULER paragraph).
 *
 *  k, v       device, dtype in_dtype (WC_F32 | WC_BF16), post-RoPE,
 *             [n_layers][n_tok][Hkv][128]; layer l starts at
 *             l * layer_stride elements.
 *  layer0     first cache layer written; layers layer0 .. layer0+n_layers-1.
 *  slot       device int64 [n_tok]: page * page_size + offset of each token
 *             (the same slots in every layer).  For 2-bit the tokens must
 *             come in whole pages: slot[32g + i] = page_g * 32 + i.
 *  pos        device int32 [n_tok]: the token's 0-based position in its
 *             sequence (dither counter).
 *  seed       device uint64 [n_tok]: dither seed of the token's sequence.
 * Writes k_codes, v_codes, scales (or aux), the key witness and, when
 * cache->v_witness is set, the value witness; in a repaired block (exact_slot
 * >= 0) the key witness is 0 and the exact key goes to the block's pool row
 * (bf16 input only when exact_slot is set); with the
 * outlier bypass (num_outliers > 0, bf16 input only) also k_outlier, reading
 * the channels of each layer from outlier_ch.  RTN INT8: code =
 * clamp(rint(x * (127/absmax)), -128, 127), x^ = s code.  16-bit store
 * (bf16 input only): k and v are stored as given (they are the scheme's
 * outputs x^) and the witnesses are set to 0; wc_witness then stores the
 * witnesses of the scheme's residuals.
 */
int wc_write_kv(const wc_cache* cache, int layer0, int n_layers, const void* k, const void* v,
                int in_dtype, int64_t n_tok, int64_t layer_stride, const int64_t* slot,
                const int32_t* pos, const uint64_t* seed, void* stream);

/*
 * wc_write_kv_pages -- wc_write_kv for whole 16-token pages (the prefill).
 *
 * The same arithmetic and outputs as wc_write_kv (dithered INT8, fp8, RTN
 * INT8; the outlier bypass and the value witness as there), for tokens that
 * fill whole pages: input token 16 i + j goes to page pages[i], offset j, at
 * position pos0[i] + j with the dither seed seed[i].  One workgroup writes a
 * whole page-head block, so every code block leaves as full-line stores.
 *
 *  k, v     device, in_dtype, [n_layers][16 n_pages][Hkv][128]; layer l at
 *           l * layer_stride elements.
 *  pages, pos0  device int32 [n_pages];  seed  device uint64 [n_pages].
 * Other schemes return WC_EUNSUPPORTED (write them with wc_write_kv).
 */
int wc_write_kv_pages(const wc_cache* cache, int layer0, int n_layers, const void* k, const void* v,
                      int in_dtype, int64_t n_pages, int64_t layer_stride, const int32_t* pages,
                      const int32_t* pos0, const uint64_t* seed, void* stream);

/*
 * wc_witness -- the black-box hook: store the witness of any scheme.
 *
 * The summary's implementation paragraph and the abstract register any
 * scheme as one tensor function x^ = f(x) and meter it through the witness
 * of its residual: w_{t,b} = ||x^_t - x_t|| over band b (witness-theorem
 * paragraph), written at the tokens' slots in cache->witness (Tier A then
 * bounds the scheme in wc_decode_attn_meter).  With the 16-bit store the
 * caller writes x^ with wc_write_kv first, then calls this with the exact
 * keys x and the same x^.
 *
 *  x, xhat    device, dtype in_dtype (WC_F32 | WC_BF16), [n_layers][n_tok][Hkv][128],
 *             layer l at l * layer_stride elements; x = exact post-RoPE keys.
 *  slot       device int64 [n_tok]: page * 16 + offset (16-token pages).
 *  values     0: x are keys, the banded key witness goes to cache->witness;
 *             1: x are values, ||x^ - x|| goes to cache->v_witness.
 * The stored value is rounded up (by a factor 1 + 2^-20) so that it never
 * falls below the exact norm.  Keys in a repaired block (exact_slot >= 0)
 * store a zero witness and their exact key x in the block's pool row (for the
 * 16-bit store this call completes a token's write there); with exact_slot
 * set, keys must be bf16.
 */
int wc_witness(const wc_cache* cache, int layer0, int n_layers, const void* x, const void* xhat, int in_dtype,
               int64_t n_tok, int64_t layer_stride, const int64_t* slot, int values, void* stream);

/*
 * wc_outlier_select -- the outlier-bypass channels of each (layer, KV head).
 *
 * For every layer l < n_layers and KV head g, the energy of channel c is
 * E_c = sum_t x[l][t][g][c]^2 accumulated in float32 in token order
 * (E <- fp32(E + fp32(x*x)); x*x is exact for bf16 input); a NaN energy
 * counts as +inf.  The m channels of largest E_c, ties to the lower channel,
 * are written in ascending order to channels[l][g][0..m-1] (the layout of
 * wc_cache.outlier_ch).  Reading of "top-m energy channels" for the outlier
 * bypass (see the cache layout notes above).
 *
 *  x        device, dtype in_dtype (WC_F32 | WC_BF16), [n_layers][n_tok][Hkv][128],
 *           layer l at l * layer_stride elements (the calibration keys).
 *  m        1..128.
 *  channels device int32 [n_layers][Hkv][m].
 */
int wc_outlier_select(const void* x, int in_dtype, int n_layers, int64_t n_tok, int num_kv_heads,
                      int64_t layer_stride, int m, int32_t* channels, void* stream);

/*
 * wc_decode_attn_meter -- fused split-KV decode attention and meter.
 *
 * One data pass over the paged cache computes, per query head h, the
 * compressed attention sum_t p~_t v^_t and the meter accumulators of the
 * WitCert summary: Tier A (Theorem 2) c_t = sm_scale * sum_b ||q_b|| w_{t,b};
 * Tier B (dithered INT8 only) c_t = sqrt(2 varsigma_t^2 log(2S/delta_loc)),
 * varsigma_t^2 = sm_scale^2 s_t^2 ||q||^2 / 12, delta_loc = delta_req/(L*H*T)
 * (||q||^2 over the channels off O with the outlier bypass);
 * aggregated by E = sum_t p~_t expm1(c_t) (improvements list: TV <=
 * min(1, (A^2-1)/2), A = 1 + E).  Repaired blocks use exact keys and c = 0.
 *
 *  q          device [B][Hq][128], q_dtype WC_F32 | WC_BF16; Hq multiple of Hkv,
 *             Hq/Hkv <= 16.
 *  page_table device int32 [B][max_pages] physical page of each logical block
 *             (< num_pages).  The cache needs num_pages >= 1 (WC_EUNSUPPORTED
 *             otherwise): a wave's prefetch past its last block requests
 *             physical page 0.
 *  ctx_len    device int32 [B]: tokens cached per sequence (<= max_pages*16).
 *  seed       device uint64 [B]: dither seed of each sequence.
 *  Repaired blocks (exact_slot >= 0) take their keys from the bf16 pool,
 *             multiplied with the query on bf16 MFMAs (exact products; an fp32
 *             query enters as three bf16 pieces that sum to it exactly).
 *  meter_mask 0, WC_METER_A or WC_METER_A|WC_METER_B (B needs dithered INT8),
 *             plus WC_METER_V for the value certificate (any scheme; needs
 *             cache->v_witness) and WC_BLOCK_CMAX for the block output mode.
 *  Schemes: dithered INT8, fp8, RTN INT8 and the 16-bit store (2-bit has
 *             no decode path).
 *             With 0 the witness is not read; output and LSE bits are the same
 *             as with the meter on.
 *  n_split    1..1024 KV splits per (sequence, KV head): split i covers blocks
 *             [i*P_b/n_split, (i+1)*P_b/n_split) of the sequence's P_b blocks.
 *  partials   device fp32 workspace [B][Hq][n_split][136]: per split
 *             (m, l, N_A, N_B, o[128], C_A, C_B, N_V, 0) with m the running
 *             max of the logits in log2 units, l = sum 2^(l2 - m),
 *             N_X = sum 2^(l2 - m) expm1(c_X), o = sum 2^(l2 - m) v^,
 *             C_X = max_t c_X (for the tanh bound) and N_V = sum 2^(l2 - m) w^V
 *             (WC_METER_V, else 0).
 *             ws_bytes >= wc_decode_workspace_bytes().
 *  block_logrisk  nullable device fp32 [B][Hq][max_pages]: natural log of
 *             sum_{t in block} exp(l_t) expm1(c_t) for the gate's tier (B if
 *             requested, else A); -inf for blocks without risk.  With
 *             WC_BLOCK_CMAX in meter_mask it receives instead max_{t in block}
 *             c_t of the gate's tier (0 for repaired blocks), the input of
 *             wc_gate_pagein_tanh.  Entries past a sequence's ceil(S/16)
 *             pages are not written.
 */
int wc_decode_attn_meter(const wc_cache* cache, int layer, const void* q, int q_dtype, int B, int Hq,
                         const int32_t* page_table, int max_pages, const int32_t* ctx_len,
                         const uint64_t* seed, float sm_scale, unsigned meter_mask, double delta_req,
                         int L, int H, int T, int n_split, float* partials, size_t ws_bytes,
                         float* block_logrisk, void* stream);

/* Bytes of the decode workspace: B * Hq * n_split * 136 * 4. */
size_t wc_decode_workspace_bytes(int B, int Hq, int n_split);

/*
 * wc_decode_load_floor -- a measurement of the decode's memory bound, not a
 * step of the method.  The summary's cost paragraph puts the certified
 * decode's cost in the bytes it reads (codes, scales, witness); this call
 * issues exactly the page loads wc_decode_attn_meter issues for the same
 * arguments (same grid, page assignment, page-table and exact-slot reads,
 * cache policies, one page in flight per wave) and does no arithmetic, so
 * its time is what HBM delivers for that access pattern.  The query, the
 * outlier side store and the value witnesses are not read.
 *
 *  meter_mask       WC_METER_A adds the witness loads (other bits as in the
 *                   decode; they add no loads).
 *  match_residency  non-zero: each workgroup reserves the LDS of the
 *                   decode's instance for this cache (meter on, bf16 query),
 *                   so as many workgroups share a CU as in the decode; zero:
 *                   no LDS (the loads alone set the residency).
 *  sink             device uint32 [1]: written only when a lane's fold of
 *                   the loaded words hits a fixed pattern; its contents mean
 *                   nothing.
 * Returns WC_EUNSUPPORTED when a layer's code array is 4 GB or more, or the
 * cache has no physical page.
 */
int wc_decode_load_floor(const wc_cache* cache, int layer, int B, int Hq, const int32_t* page_table,
                         int max_pages, const int32_t* ctx_len, int n_split, unsigned meter_mask,
                         int match_residency, uint32_t* sink, void* stream);


/*
 * wc_lse_merge -- merge KV-split partials by log-sum-exp (output and
 * certificate together; summary implementation paragraph and paperswithlean
 * Figure 2 caption).
 *
 *  o        device fp32 [B][Hq][128]: sum_t p~_t v^_t.
 *  lse      device fp32 [B][Hq]: natural-log LSE of the logits (-inf if empty).
 *  meter_a, meter_b  nullable device fp32 [B][Hq]: R = E (1 + E/2), unclamped;
 *           the TV bound is min(1, R).  meter_b is 0 when Tier B is off.
 *  tanh_a, tanh_b    nullable device fp32 [B][Hq]: the deterministic tanh
 *           bound tanh(max_t c_t / 2) of each tier, which the summary's
 *           page-in paragraph compares the certificate with (the pages give
 *           no formula; this is the bound for logits that each move by at
 *           most c_t: the log-ratio of the two softmaxes then spans at most
 *           2 max c, and a span D gives TV <= tanh(D/4)).  0 when the tier
 *           is off or the sequence is empty.
 *  meter_v  nullable device fp32 [B][Hq]: the value certificate E_V (0 when
 *           WC_METER_V was off).
 */
int wc_lse_merge(const float* partials, int B, int Hq, int n_split, float* o, float* lse,
                 float* meter_a, float* meter_b, float* tanh_a, float* tanh_b, float* meter_v, void* stream);

/*
 * wc_gate_pagein -- meter-driven repair from the exact backing store.
 *
 * WitCert summary (implementation paragraph) and paperswithlean
 * (Problem/Approach, Figure 2 and Figure 5 captions): when the meter exceeds
 * tau, exact blocks are paged in from the CPU store, ranked by risk, the
 * repaired witnesses are zeroed and the repair persists.  Per (sequence b,
 * KV head g): rho_fx[h][j] = min(ceil(exp(logrisk - lse_h) * 2^40), 2^47);
 * X_h = sum_j rho_fx; trigger when max_h X_h > T = floor((sqrt(1+2 tau)-1) 2^40);
 * repair the shortest prefix of the unrepaired blocks ranked by
 * max_h rho_fx[h][j] (ties to the lower index) that leaves every
 * X_h - sum rho_fx <= T, capped by budget_blocks (-1 = no cap).  Pool slots
 * are handed out in (b, g, rank) order from *pool_used; selection stops when
 * the pool is full.
 *
 *  meter         nullable device fp32 [B][Hq]: the merged meter R of the same
 *                tier as block_logrisk (R_B of a Tier B decode, else R_A), as
 *                wc_lse_merge returns it with this lse.  A pair (b, g) whose
 *                heads all have E = 2R / (sqrt(1 + 2R) + 1) with
 *                E (1 + 2^-10) + (P_b + 1) 2^-39 <= E_tau cannot trigger (X_h
 *                is that sum taken per block, each rounded up by < 2^-40), and
 *                skips the pass over its block risks; the decisions are the
 *                same as with meter = NULL.  Ignored when rho_fx is given.
 *  host_exact_k  pinned host bf16 [L][P][Hkv][16][128], device-readable
 *                (hipHostMalloc / torch pin_memory); a pointer the device
 *                cannot map returns WC_EINVAL before any launch.  It holds
 *                the exact keys of every token written so far; the pool rows
 *                of tokens appended after a repair are written by the write
 *                path.
 *  pool_used     device int64 [1], in/out.
 *  bytes_paged   device int64 [1], incremented by 4096 per repaired block.
 *  selected      nullable device int32 [B][Hkv][max_pages + 1]: count, then
 *                the chosen blocks in rank order (those that got a slot).
 *  rho_fx        nullable device uint64 [B][Hq][max_pages] test export.
 *  workspace     device scratch, ws_bytes >= wc_gate_workspace_bytes().
 * Requires cache->exact_slot and exact_pool; 0 <= tau, E_tau < 64;
 * max_pages <= 65536 (sequences of up to 1,048,576 tokens).  A triggered
 * (sequence, KV head) sorts its candidate blocks in LDS tiles of 4096 and
 * merges the tiles in the workspace, so any length up to that bound is ranked
 * exactly.
 */
int wc_gate_pagein(const wc_cache* cache, int layer, const float* block_logrisk, const float* lse,
                   const float* meter, int B, int Hq, const int32_t* page_table, int max_pages, const int32_t* ctx_len,
                   double tau, int64_t budget_blocks, const uint16_t* host_exact_k,
                   int64_t* pool_used, int64_t* bytes_paged, int32_t* selected, uint64_t* rho_fx,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * wc_gate_pagein_noalloc -- wc_gate_pagein for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, checks, kernels and outputs, without the
 * workspace.  Its scratch (the workspace wc_gate_pagein takes) is a static
 * device array of WC_GATE_NOALLOC_MAX_BYTES in the library, one copy per GPU,
 * held until the process ends; its device address is looked up once per
 * device, on the first call with that device current.  A call whose
 * wc_gate_workspace_bytes(B, Hkv, max_pages) exceeds the array returns
 * WC_EWORKSPACE before any launch.  The call allocates nothing (no hipMalloc,
 * no hipFree).  Every call on one GPU shares its array: calls that overlap on
 * one GPU (different streams or threads without ordering) race; calls ordered
 * on one stream do not (each call writes everything it later reads).
 */
#define WC_GATE_NOALLOC_MAX_BYTES ((size_t)16 << 20)
int wc_gate_pagein_noalloc(const wc_cache* cache, int layer, const float* block_logrisk, const float* lse,
                           const float* meter, int B, int Hq, const int32_t* page_table, int max_pages,
                           const int32_t* ctx_len, double tau, int64_t budget_blocks, const uint16_t* host_exact_k,
                           int64_t* pool_used, int64_t* bytes_paged, int32_t* selected, uint64_t* rho_fx,
                           void* stream);

/* Bytes of the gate workspace for B sequences, Hkv heads and max_pages blocks:
 * the selection (4 B per block), the counts, the pool counter and two sort
 * buffers (8 B per block each). */
size_t wc_gate_workspace_bytes(int B, int Hkv, int max_pages);

/*
 * wc_gate_pagein_tanh -- the tanh gate the certificate is compared with
 * (summary, page-in paragraph: the certificate pages in less than the
 * deterministic tanh bound).  tanh(max_t c_t / 2) <= tau for every head
 * exactly when no unrepaired token has c_t > c* = 2 artanh(tau) (c* = +inf
 * for tau >= 1), so per (sequence b, KV head g) it repairs every unrepaired
 * block j with max_h block_cmax[b][h][j] > c* (float32 comparison), ranked
 * by that value (descending, ties to the lower index), capped by
 * budget_blocks; pool slots, page-in, witness zeroing and `selected` are as
 * in wc_gate_pagein.
 *
 *  block_cmax  device fp32 [B][Hq][max_pages]: the decode's block output
 *              with WC_BLOCK_CMAX.
 *  workspace   as for wc_gate_pagein (wc_gate_workspace_bytes()).
 * Requires cache->exact_slot and exact_pool; tau >= 0; max_pages <= 65536;
 * host_exact_k as for wc_gate_pagein.
 */
int wc_gate_pagein_tanh(const wc_cache* cache, int layer, const float* block_cmax, int B, int Hq,
                        const int32_t* page_table, int max_pages, const int32_t* ctx_len, double tau,
                        int64_t budget_blocks, const uint16_t* host_exact_k, int64_t* pool_used,
                        int64_t* bytes_paged, int32_t* selected, void* workspace, size_t ws_bytes, void* stream);

/*
 * wc_dither_fill -- test hook: the 16-bit dither draws k (xi = k/65536 - 1/2)
 * the kernels regenerate for positions pos0 .. pos0+n_pos-1 of one (sequence
 * seed, layer, KV head), into device uint16 out[n_pos][128].  The draw is a
 * counter hash of (seed, layer, head, token, channel) (summary, Tier B
 * paragraph): keys and values at one (token, channel) share it.
 */
int wc_dither_fill(uint64_t seed, int layer, int kv_head, int64_t pos0, int64_t n_pos, uint16_t* out,
                   void* stream);

const char* wc_last_error(void);
const char* wc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WITCERT_H */
