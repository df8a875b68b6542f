"""moe_dispatch_noalloc, the entry point for callers that cannot allocate (its histogram lives in
the library's fixed device array), against moe_dispatch with a caller's workspace (needs an
MI355X).  Integer outputs, so bit-exact; two calls in a row, the second with a smaller input, so
that the second call runs on the array the first one left behind."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from sparse_mixture_experts_counting_amd import build
    import os
    if not os.path.exists(build.LIB):
        build.build()
    from sparse_mixture_experts_counting_amd import layer, libmoe, synth
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return dict(layer=layer, lm=libmoe, synth=synth)


def _topk(T, E, k, seed):
    rng = np.random.default_rng(seed)
    L = rng.normal(size=(T, E)) - 0.4 * np.log1p(np.arange(E))[None, :]   # skewed loads
    return np.argsort(-L, axis=1, kind="stable")[:, :k].astype(np.int32)


def _run(M, idx, E, C, noalloc):
    lm = M["lm"]
    T, k = idx.shape
    dev = torch.device("cuda")
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
               perm=torch.full((T * k,), -7, **i32), inv=torch.full((T * k,), -7, **i32),
               n_dropped=torch.full((1,), -7, **i32))
    topk = torch.from_numpy(idx).to(dev)
    if noalloc:
        lm.dispatch_noalloc(topk, T, E, k, C, out["counts"], out["offsets"], out["perm"],
                            out["inv"], out["n_dropped"])
    else:
        ws = torch.empty(M["lm"].lib().moe_workspace_bytes(T, 8, 8, E, k, 0), dtype=torch.uint8,
                         device=dev)
        lm.dispatch(topk, T, E, k, C, out["counts"], out["offsets"], out["perm"], out["inv"],
                    out["n_dropped"], ws)
    torch.cuda.synchronize()
    res = {n: t.cpu().numpy() for n, t in out.items()}
    res["perm"] = res["perm"][: int(res["offsets"][-1])]
    return res


@pytest.mark.parametrize("first,second", [((8192, 256, 8, 0), (300, 256, 8, 20)),
                                          ((60000, 1024, 4, 250), (2048, 8, 1, 256)),
                                          ((4096, 8, 2, 600), (33, 8, 2, 5))])
def test_noalloc_matches_workspace_dispatch(M, first, second):
    for n, (T, E, k, C) in enumerate((first, second)):
        print("dispatch_noalloc call %d: T=%d E=%d k=%d C=%d" % (n, T, E, k, C), flush=True)
        idx = _topk(T, E, k, seed=T + E)
        want = _run(M, idx, E, C, noalloc=False)
        got = _run(M, idx, E, C, noalloc=True)
        for name in ("counts", "offsets", "perm", "inv", "n_dropped"):
            np.testing.assert_array_equal(got[name], want[name], err_msg=name)
        if C > 0:
            assert want["n_dropped"][0] > 0


def test_noalloc_rejects_beyond_its_array(M):
    """More assignments than the 1 MiB histogram array holds: refused before any launch."""
    lm = M["lm"]
    T, E, k = 600000, 1024, 1                    # 293 chunks x 1024 experts x 4 B > 1 MiB
    dev = torch.device("cuda")
    small = torch.zeros(16, dtype=torch.int32, device=dev)
    with pytest.raises(lm.MoEError) as ei:
        lm.dispatch_noalloc(small, T, E, k, 0, small, small, small, small, small)
    assert ei.value.status == 2
