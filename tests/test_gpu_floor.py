"""The decode's load floor (a measurement hook): it runs on every scheme the
decode serves, on ragged batches with empty sequences, with and without the
decode's LDS reservation, and writes nothing but its one-word sink."""
import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from tests import helpers as H
from tests.scenario import Scenario

pytestmark = pytest.mark.gpu


def _mantissa4(bits):
    b = bits.astype(np.uint32)
    return (((b + 0x4) & 0xFFF8) & 0xFFFF).astype(np.uint16)


@pytest.mark.parametrize("scheme", ["int8", "fp8", "rtn", "store16"])
@pytest.mark.parametrize("Hq", [28, 64])
def test_load_floor_runs_and_writes_only_its_sink(scheme, Hq):
    L = H.need_gpu()
    print(f"load floor {scheme} Hq={Hq}", flush=True)
    lens = [1, 0, 700, 33]
    n = sum(lens)
    d = inputs.layer(seed=60, S=n, Hq=Hq, Hkv=4, outliers=0)
    q = inputs.layer(seed=61, S=1, Hq=Hq, Hkv=4, batch=len(lens))["q"]
    sch = {"int8": L.WC_DITHER_INT8, "fp8": L.WC_FP8_E4M3, "rtn": L.WC_RTN_INT8, "store16": L.WC_BF16_STORE}[scheme]
    kw = dict(khat=_mantissa4(d["k"][:n]), vhat=_mantissa4(d["v"][:n])) if scheme == "store16" else {}
    sc = Scenario(sch, d["k"][:n], d["v"][:n], q, lens, "bf16", Hkv=4, **kw)
    before = sc.decode(n_split=3, mask=1)
    k_codes = sc.cache.k_codes.clone()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for mask in (0, 1):
        for match in (True, False):
            for ns in (1, 5):
                L.wc_decode_load_floor(sc.cache, sc.layer, Hq, sc.dev["tab"], sc.dev["ctx"], ns, mask, sink,
                                       match_residency=match)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF in (0, 0x9E3779B9)
    assert torch.equal(k_codes, sc.cache.k_codes)
    after = sc.decode(n_split=3, mask=1)
    for key in ("o", "lse", "R_A"):
        assert np.array_equal(after[key].view(np.uint32), before[key].view(np.uint32)), key
