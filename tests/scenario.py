"""One decode scenario run through the C ABI and through the oracle.

Used by the GPU parity tests: write K/V with wc_write_kv, decode with
wc_decode_attn_meter, merge with wc_lse_merge; the oracle quantizes the same
inputs and evaluates the same attention and meter in float64.
"""
import math

import numpy as np
import torch

from certified_kv_cache_amd import inputs
from oracle import meter, outlier, quant
from tests import helpers as H


class Scenario:
    def __init__(self, scheme, k, v, q, ctx_lens, dtype, Hkv, layer=1, num_layers=2, seed=5, pool_capacity=0,
                 extra_pages=3, delta=(1e-2, 28, 28, 256), num_outliers=0, khat=None, vhat=None, v_witness=False):
        from certified_kv_cache_amd import _lib as L
        self.L = L
        self.scheme, self.dtype, self.Hkv = scheme, dtype, Hkv
        self.ctx = np.asarray(ctx_lens, dtype=np.int64)
        self.B, self.Hq = q.shape[0], q.shape[1]
        self.G = self.Hq // Hkv
        self.layer = layer
        self.delta = delta
        self.tab, self.num_pages = inputs.page_table(seed, self.ctx, extra_pages=extra_pages)
        self.seeds = inputs.seeds(self.B, base=1000 + seed)
        self.k, self.v, self.q = k, v, q
        self.cache = L.KVCache(scheme, num_layers, self.num_pages, Hkv, pool_capacity=pool_capacity,
                               num_outliers=num_outliers, v_witness=v_witness)
        # outlier bypass: the oracle's top-energy channels over all cached keys of each head
        self.bypass = None
        if num_outliers:
            k32 = H.to_f32(k, dtype)
            self.bypass = np.stack([outlier.top_energy_channels(k32[:, g], num_outliers) for g in range(Hkv)])
            self.cache.outlier_ch[layer] = torch.from_numpy(self.bypass).cuda()
        slot, pos, seq = H.slots_for(self.tab, self.ctx)
        self.dev = dict(
            slot=torch.from_numpy(slot).cuda(), pos=torch.from_numpy(pos).cuda(),
            tseed=torch.from_numpy(self.seeds[seq].view(np.int64)).cuda(),
            seed=torch.from_numpy(self.seeds.view(np.int64)).cuda(),
            tab=torch.from_numpy(self.tab).cuda(), ctx=torch.from_numpy(self.ctx.astype(np.int32)).cuda(),
            q=H.dev_tensor(q, dtype))
        # 16-bit store: a black-box scheme's outputs khat, vhat (bf16 bits) are
        # stored, and the witness of khat against k comes from wc_witness
        self.khat, self.vhat = khat, vhat
        if len(slot):
            if scheme == L.WC_BF16_STORE:
                L.wc_write_kv(self.cache, H.dev_tensor(khat, dtype), H.dev_tensor(vhat, dtype), self.dev["slot"],
                              self.dev["pos"], self.dev["tseed"], layer0=layer)
                L.wc_witness(self.cache, H.dev_tensor(k, dtype), H.dev_tensor(khat, dtype), self.dev["slot"],
                             layer0=layer)
                if v_witness:
                    L.wc_witness(self.cache, H.dev_tensor(v, dtype), H.dev_tensor(vhat, dtype), self.dev["slot"],
                                 layer0=layer, values=True)
            else:
                L.wc_write_kv(self.cache, H.dev_tensor(k, dtype), H.dev_tensor(v, dtype), self.dev["slot"],
                              self.dev["pos"], self.dev["tseed"], layer0=layer)
        self.offsets = np.concatenate([[0], np.cumsum(self.ctx)])

    def decode(self, n_split=4, mask=3, risk=False, sm=H.SM, cmax=False, vcert=False):
        L = self.L
        B, Hq = self.B, self.Hq
        part = torch.empty(L.wc_decode_workspace_bytes(B, Hq, n_split) // 4, dtype=torch.float32, device="cuda")
        br = torch.full((B, Hq, self.tab.shape[1]), float("nan"), device="cuda") if (risk or cmax) else None
        L.wc_decode_attn_meter(self.cache, self.layer, self.dev["q"], self.dev["tab"], self.dev["ctx"],
                               self.dev["seed"], part, sm,
                               mask | (L.WC_BLOCK_CMAX if cmax else 0) | (L.WC_METER_V if vcert else 0), self.delta[0],
                               *self.delta[1:], n_split, block_logrisk=br)
        o = torch.empty((B, Hq, 128), device="cuda")
        lse = torch.empty((B, Hq), device="cuda")
        ra, rb, ta, tb, ev = (torch.empty((B, Hq), device="cuda") for _ in range(5))
        L.wc_lse_merge(part, B, Hq, n_split, o, lse, ra, rb, ta, tb, ev)
        torch.cuda.synchronize()
        out = dict(o=o.cpu().numpy(), lse=lse.cpu().numpy(), R_A=ra.cpu().numpy(), R_B=rb.cpu().numpy(),
                   T_A=ta.cpu().numpy(), T_B=tb.cpu().numpy(), E_V=ev.cpu().numpy(), part=part.cpu().numpy())
        if risk:
            out["logrisk"] = br.cpu().numpy()
        if cmax:
            out["cmax"] = br.cpu().numpy()
        return out

    def seq_inputs(self, b, g):
        s0, s1 = self.offsets[b], self.offsets[b + 1]
        k32 = H.to_f32(self.k[s0:s1, g], self.dtype)
        v32 = H.to_f32(self.v[s0:s1, g], self.dtype)
        q = H.to_f32(self.q[b, g * self.G:(g + 1) * self.G], self.dtype).astype(np.float64)
        return k32, v32, q

    def oracle(self, b, g, repaired=None, sm=H.SM):
        S = int(self.ctx[b])
        k32, v32, q = self.seq_inputs(b, g)
        if self.scheme == self.L.WC_DITHER_INT8:
            O = None if self.bypass is None else self.bypass[g]
            oc = H.oracle_int8_cache(k32, v32, int(self.seeds[b]), self.layer, g, S, bypass=O)
            dl = meter.delta_loc(*self.delta)
            lt = math.log(2 * S / dl) if S > 0 else 0.0
            res = meter.decode_group(q, k32, oc["khat"], v32, oc["vhat"], oc["w"], sm, k_scale=oc["sk"],
                                     log_term=lt, repaired=repaired, bypass=O)
        elif self.scheme == self.L.WC_RTN_INT8:
            oc = H.oracle_rtn_cache(k32, v32)
            res = meter.decode_group(q, k32, oc["khat"], v32, oc["vhat"], oc["w"], sm, repaired=repaired)
        elif self.scheme == self.L.WC_BF16_STORE:
            s0, s1 = self.offsets[b], self.offsets[b + 1]
            kh = H.to_f32(self.khat[s0:s1, g], self.dtype)
            vh = H.to_f32(self.vhat[s0:s1, g], self.dtype)
            oc = dict(khat=kh, vhat=vh, w=quant.witness(k32, kh))
            res = meter.decode_group(q, k32, kh, v32, vh, oc["w"], sm, repaired=repaired)
        else:
            oc = H.oracle_fp8_cache(k32, v32)
            res = meter.decode_group(q, k32, oc["khat"], v32, oc["vhat"], oc["w"], sm, repaired=repaired)
        return oc, res
