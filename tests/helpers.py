"""Test plumbing: device handling, cache-layout gathers, oracle pipelines.

Gathers only re-index the library's documented HBM layouts into logical
[token, ...] arrays; the arithmetic lives in oracle/ and in the HIP library.
"""
import math

import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import dither, meter, outlier, quant

SM = 1.0 / math.sqrt(128)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from certified_kv_cache_amd import _lib  # noqa: F401  (fails loudly if not built)
    return _lib


def to_f32(a, dtype):
    """Exact float32 view of a synthesized input (bf16 bits or float32)."""
    return inputs.bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


def dev_tensor(a, dtype, device="cuda"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def slots_for(page_table, ctx_lens, page_size=16):
    """slot (page*ps + offset), position and sequence index of every cached token, in sequence order."""
    slots, pos, seq = [], [], []
    for b, S in enumerate(ctx_lens):
        t = np.arange(S)
        slots.append(page_table[b, t // page_size].astype(np.int64) * page_size + t % page_size)
        pos.append(t.astype(np.int32))
        seq.append(np.full(S, b))
    return np.concatenate(slots), np.concatenate(pos), np.concatenate(seq)


def gather_k_codes(kc, layer, pt_row, S, g):
    """[S, 128] key codes of one sequence and KV head from [L][P][Hkv][2][4][16][16]:
    token t, channel c at [(c % 32) // 16][c // 32][t % 16][c % 16]."""
    t = np.arange(S)[:, None]
    c = np.arange(128)[None, :]
    return kc[layer, pt_row[t // 16], g, (c % 32) // 16, c // 32, t % 16, c % 16]


def gather_v_codes(vc, layer, pt_row, S, g):
    """[S, 128] value codes from [L][P][Hkv][2][4][16][4][4]: token t, channel c
    at [(c % 32) // 16][(t % 16) // 4][4 (c // 32) + c % 4][(c % 16) // 4][t % 4]."""
    t = np.arange(S)[:, None]
    c = np.arange(128)[None, :]
    return vc[layer, pt_row[t // 16], g, (c % 32) // 16, (t % 16) // 4, 4 * (c // 32) + c % 4, (c % 16) // 4, t % 4]


def gather_k_bf16(kc, layer, pt_row, S, g):
    """[S, 128] bf16 bits of the 16-bit store's keys from [L][P][Hkv][4][4][16][8]:
    token t, channel c at [(c % 32) // 8][c // 32][t % 16][c % 8]."""
    t = np.arange(S)[:, None]
    c = np.arange(128)[None, :]
    return kc[layer, pt_row[t // 16], g, (c % 32) // 8, c // 32, t % 16, c % 8]


def gather_v_bf16(vc, layer, pt_row, S, g):
    """[S, 128] bf16 bits of the 16-bit store's values from [L][P][Hkv][4][4][16][2][4]:
    token t, channel c at [(c % 8) // 2][(t % 16) // 4][c // 8][c % 2][t % 4]."""
    t = np.arange(S)[:, None]
    c = np.arange(128)[None, :]
    return vc[layer, pt_row[t // 16], g, (c % 8) // 2, (t % 16) // 4, c // 8, c % 2, t % 4]


def gather_rows(arr, layer, pt_row, S, g):
    """[S, ...] per-token rows (scales, witness) from [L][P][Hkv][16][...]."""
    t = np.arange(S)
    return arr[layer, pt_row[t // 16], g, t % 16]


def oracle_int8_cache(k32, v32, seed, layer, g, S, bypass=None):
    """Oracle write of one (sequence, KV head): codes, scales, dequantized, witness.

    bypass: outlier-bypass channels of the keys (their exact values in "side")."""
    pos = np.arange(S)
    xk = xv = dither.dither_rows(seed, layer, g, pos)
    if bypass is not None and len(bypass):
        ck, sk, _, side = outlier.dither_int8_bypass(k32, xk, bypass)
        khat = outlier.dequant_bypass(ck, sk, xk, side, bypass)
    else:
        ck, sk, _ = quant.dither_int8(k32, xk)
        khat = quant.dequant_dither_int8(ck, sk, xk)
        side = None
    cv, sv, _ = quant.dither_int8(v32, xv)
    vhat = quant.dequant_dither_int8(cv, sv, xv)
    return dict(ck=ck, sk=sk, cv=cv, sv=sv, khat=khat, vhat=vhat, w=quant.witness(k32, khat), side=side)


def oracle_rtn_cache(k32, v32):
    ck, sk, _ = quant.rtn_int8(k32)
    cv, sv, _ = quant.rtn_int8(v32)
    khat = quant.dequant_rtn_int8(ck, sk)
    return dict(ck=ck, sk=sk, cv=cv, sv=sv, khat=khat, vhat=quant.dequant_rtn_int8(cv, sv),
                w=quant.witness(k32, khat))


def oracle_fp8_cache(k32, v32):
    ck, kval = quant.fp8_e4m3(k32)
    cv, vval = quant.fp8_e4m3(v32)
    return dict(ck=ck, cv=cv, khat=kval, vhat=vval, w=quant.witness(k32, kval), sk=None)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-300)
