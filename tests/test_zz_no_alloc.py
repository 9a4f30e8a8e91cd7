"""wushkv_decode_step_noalloc (the decode step whose workspace is the
library's per-GPU scratch array) against wushkv_decode_step with a caller
workspace: two identical caches take the same steps, one through each entry
point, on two calls in a row, the second with a smaller input (fewer
sequences).  Outputs must be bit-identical and within the oracle bar, and the
caches left behind identical."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_wushkv_amd import synth, wushkv_decode_step_noalloc
from decode_attention_wushkv_amd.device_cache import DeviceCache

from cachepack import read_unit
from gpu_checks import check_attention, reference_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_wushkv_amd import build
    if build.is_stale():
        build.build()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("G,n_kv,L0s", [(4, 8, [1500, 0, 777]), (1, 2, [3000, 1200, 640])])
def test_noalloc_step_equals_decode_step(G, n_kv, L0s):
    w = synth.Workload(14, "noalloc", 1, n_kv * G, n_kv, len(L0s), max(L0s) + 2, (2,), 4, 128, 1,
                       0.01, 0.99, "bf16")
    lengths = [L + 2 for L in L0s]
    T, Tq = synth.transforms(w, 0)
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    ks, vs = zip(*[synth.keys_values(w, 0, si, 0, L) for si, L in enumerate(lengths)])
    caches = []
    slots = list(range(len(L0s)))
    for _ in range(2):
        dc = DeviceCache(n_layers=1, n_q_heads=w.n_q, n_kv_heads=n_kv, bits=2, sink=4, recent=128,
                         max_batch=len(L0s), ctx_cap=max(lengths), io_dtype=torch.bfloat16,
                         device="cuda")
        kk = torch.cat([ks[i][:L0s[i]] for i in slots]).cuda().contiguous()
        vv = torch.cat([vs[i][:L0s[i]] for i in slots]).cuda().contiguous()
        dc.append(0, slots, L0s, kk, vv, tk)
        caches.append(dc)
    a, b = caches
    pos = list(L0s)
    # call 1: every sequence; call 2: a smaller input (one sequence)
    for call, sl in enumerate([slots, [slots[-1]]]):
        k1 = torch.stack([ks[i][pos[i]] for i in sl]).cuda().contiguous()
        v1 = torch.stack([vs[i][pos[i]] for i in sl]).cuda().contiguous()
        q = synth.queries(w, 0, call, len(sl))
        qd = q.cuda()
        out_a = a.decode_step(0, sl, k1, v1, tk, qd, tq)
        out_b = torch.full_like(out_a, float("nan"))
        wushkv_decode_step_noalloc(b.handle, 0, sl, k1.data_ptr(), v1.data_ptr(), tk.data_ptr(),
                                   qd.data_ptr(), tq.data_ptr(), out_b.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"call {call}: outputs differ"
        got = out_b.cpu().numpy()
        for j, si in enumerate(sl):
            Lq = pos[si] + 1
            units = {h: oracle.cache_unit(ks[si][:Lq, h].double().numpy(),
                                          vs[si][:Lq, h].double().numpy(),
                                          T[h].astype(np.float64), S=4, R=129, F=1, bits=2,
                                          p_lo=0.01, p_hi=0.99)
                     for h in range(n_kv)}
            check_attention(got[j], reference_attention(w, T, q[j], units))
        for si in sl:
            pos[si] += 1
    for si in slots:
        assert a.get_len(0, si) == b.get_len(0, si)
        for h in range(n_kv):
            ua = read_unit(a, 0, si, h, pos[si])
            ub = read_unit(b, 0, si, h, pos[si])
            sq = ua["squant"]
            for key in ("kcodes", "vcodes", "ks16", "kz16", "vs16", "vz16"):
                assert np.array_equal(ua[key][4:sq], ub[key][4:sq]), key
            for key in ("kwin", "vwin"):
                assert np.array_equal(np.nan_to_num(ua[key], nan=7.0), np.nan_to_num(ub[key], nan=7.0))
    a.close()
    b.close()
