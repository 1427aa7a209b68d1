"""The allocation-free gate entry point against wc_gate_pagein.

wc_gate_pagein_noalloc runs the same kernels as wc_gate_pagein with the
workspace in a static device array.  Two calls in a row (the second on a
smaller batch, so the array still holds the first call's contents) must give
exactly what wc_gate_pagein gives on identical caches: selections, exported
fixed-point risks, pool slots and contents, zeroed witnesses, counters.  A
call that needs more scratch than the array holds is refused before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from tests import helpers as H
from tests.scenario import Scenario

pytestmark = pytest.mark.gpu

CASES = [([300, 1000, 64, 700, 2000], 91, 0.05), ([129, 40], 92, 0.02)]


def _prepare(L, lens, seed):
    n = int(sum(lens))
    d = inputs.layer(seed=seed, S=n, Hq=28, Hkv=4, outliers=2)
    q = inputs.layer(seed=seed + 1, S=1, batch=len(lens))["q"]
    sc = Scenario(L.WC_DITHER_INT8, d["k"], d["v"], q, lens, "bf16", Hkv=4, pool_capacity=4096)
    store = np.zeros((2, sc.num_pages, 4, 16, 128), dtype=np.uint16)
    for b, S in enumerate(lens):
        t = np.arange(S)
        store[sc.layer, sc.tab[b, t // 16], :, t % 16] = d["k"][sc.offsets[b]:sc.offsets[b + 1]]
    host = torch.from_numpy(store.view(np.int16)).pin_memory()
    out = sc.decode(n_split=4, mask=3, risk=True)
    return sc, host, out


def _gate(L, sc, host, out, tau, noalloc):
    B, Hq, mp = sc.B, sc.Hq, sc.tab.shape[1]
    pool_used = torch.full((1,), 3, dtype=torch.int64, device="cuda")     # slots 0..2 already taken
    paged = torch.full((1,), 12288, dtype=torch.int64, device="cuda")
    sel = torch.full((B, 4, mp + 1), -7, dtype=torch.int32, device="cuda")
    rho = torch.zeros((B, Hq, mp), dtype=torch.int64, device="cuda")
    args = (sc.cache, sc.layer, torch.from_numpy(out["logrisk"]).cuda(), torch.from_numpy(out["lse"]).cuda(),
            sc.dev["tab"], sc.dev["ctx"], tau, host, pool_used, paged)
    if noalloc:
        L.wc_gate_pagein_noalloc(*args, selected=sel, rho_fx=rho)
    else:
        ws = torch.empty(L.wc_gate_workspace_bytes(B, 4, mp), dtype=torch.uint8, device="cuda")
        L.wc_gate_pagein(*args, ws, selected=sel, rho_fx=rho)
    return pool_used, paged, sel, rho


def _snapshot(sc, res):
    torch.cuda.synchronize()
    pool_used, paged, sel, rho = res
    return dict(pool_used=pool_used.cpu().numpy(), paged=paged.cpu().numpy(), sel=sel.cpu().numpy(),
                rho=rho.cpu().numpy(), slot=sc.cache.exact_slot.cpu().numpy(),
                pool=sc.cache.exact_pool.view(torch.int16).cpu().numpy(), wit=sc.cache.witness.cpu().numpy())


def test_noalloc_gate_equals_the_workspace_gate_on_two_calls():
    L = H.need_gpu()
    print("noalloc gate: two calls in a row, then the workspace gate on identical caches", flush=True)
    runs = {}
    for noalloc in (True, False):
        prepared = [_prepare(L, lens, seed) for lens, seed, _ in CASES]
        for (lens, seed, tau), (sc, host, out) in zip(CASES, prepared):
            runs[(noalloc, seed)] = _snapshot(sc, _gate(L, sc, host, out, tau, noalloc))
    for _, seed, _ in CASES:
        a, b = runs[(True, seed)], runs[(False, seed)]
        for key in a:
            assert np.array_equal(a[key], b[key]), (seed, key)
        assert int(a["pool_used"][0]) > 3, seed            # something was repaired
        print(f"  seed {seed}: {int(a['pool_used'][0]) - 3} blocks paged in, identical", flush=True)


def test_noalloc_gate_refuses_more_than_its_scratch():
    L = H.need_gpu()
    print("noalloc gate: oversize request", flush=True)
    sc, host, out = _prepare(L, [300, 64], 93)
    p = ctypes.c_void_p(16)
    mp = 65536
    need = L.wc_gate_workspace_bytes(64, 4, mp)
    assert need > L.GATE_NOALLOC_MAX_BYTES
    rc = L.lib.wc_gate_pagein_noalloc(sc.cache.ref(), sc.layer, p, p, None, 64, 28, p, mp, p, 0.2, -1,
                                      ctypes.c_void_p(host.data_ptr()), p, p, None, None, None)
    assert rc == L.WC_EWORKSPACE and b"scratch" in L.lib.wc_last_error()
