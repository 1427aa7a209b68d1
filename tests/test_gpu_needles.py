"""GPU parity on the structured variant (a sink and planted needle keys that
concentrate attention): the lazy rescale and the meters on peaked softmaxes."""
import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from tests import helpers as H
from tests.scenario import Scenario

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("scheme", ["int8", "fp8"])
def test_needle_workload_parity(scheme):
    L = H.need_gpu()
    print(f"needles {scheme}", flush=True)
    lens = [900, 2000]
    n = sum(lens)
    d = inputs.layer(seed=97, S=n, outliers=2)
    q = inputs.layer(seed=98, S=1, batch=2)["q"]
    # plant per sequence: the generator works on a [batch*S] layout of equal lengths,
    # so each sequence is planted on its own
    kt = torch.from_numpy(d["k"].view(np.int16)).view(torch.bfloat16)
    qt = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16)
    parts, o = [], 0
    for b, S in enumerate(lens):
        parts.append(inputs.plant_needles_torch(kt[o:o + S], qt[b:b + 1], 1, S, Hkv=4, seed=b))
        o += S
    k = torch.cat(parts).view(torch.int16).numpy().view(np.uint16)
    sch = L.WC_DITHER_INT8 if scheme == "int8" else L.WC_FP8_E4M3
    sc = Scenario(sch, k, d["v"][:n], q, lens, "bf16", Hkv=4)
    mask = 3 if scheme == "int8" else 1
    for n_split in (1, 7):
        out = sc.decode(n_split=n_split, mask=mask, risk=True)
        for b, S in enumerate(lens):
            for g in range(4):
                _, r = sc.oracle(b, g)
                hs = slice(g * 7, (g + 1) * 7)
                assert np.max(r["p_tilde"]) > 0.05                        # attention is concentrated
                assert np.all(H.rel_l2(out["o"][b, hs], r["o_tilde"]) <= 2e-3), (b, g)
                assert np.all(np.abs(out["lse"][b, hs] - r["lse"]) <= 1e-4 * np.maximum(1, np.abs(r["lse"])))
                for key in ("R_A", "T_A") + (("R_B", "T_B") if scheme == "int8" else ()):
                    slack = 1e-7 if key[0] == "T" else 0.0
                    assert np.all(np.abs(out[key][b, hs] - r[key]) <= 1e-4 * r[key] + slack), (key, b, g)
                assert np.all(out["R_A"][b, hs] >= r["tv_true"])
                P = -(-S // 16)
                rho = np.exp(out["logrisk"][b, hs, :P].astype(np.float64) - out["lse"][b, hs, None])
                assert np.all(np.abs(rho - r["block_risk"]) <= 1e-4 * r["block_risk"] + 1e-30), (b, g)
