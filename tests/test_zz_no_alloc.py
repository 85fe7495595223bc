"""GPU test of sparse_ffn_forward_noalloc (through the C ABI): the forward whose workspace
is the library's fixed device scratch gives the same y and the same TwELL + backup, bit for
bit, as sparse_ffn_forward with a caller workspace, on two calls in a row (the second with
fewer tokens), and refuses a call whose workspace would not fit the scratch."""
import numpy as np
import pytest

from gen import CONFIGS, make_layer
from tests.gpu_helpers import layer_to_dev, need_gpu

pytestmark = pytest.mark.gpu

KEYS = ("counts", "vals", "cols", "bk_tile", "bk_tok", "bk_vals", "bk_tile_ptr")


def _cfg(sffn, T, c, cap):
    return sffn.Config(d_model=c.D, d_ff=c.F, tile=c.tile, ell_width=c.ell_width,
                       max_tokens=T, backup_capacity=cap, dtype=c.dtype)


@pytest.mark.parametrize("name,rho,Ts", [("C3", 0.05, (300, 100)), ("C4", None, (600, 37)),
                                         ("C2", None, (4096, 1000))])
def test_noalloc_matches_forward(name, rho, Ts):
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS[name], seed=0, T=Ts[0], rho=rho)
    c = L["cfg"]
    cfg = _cfg(sffn, Ts[0], c, cap=c.n_tiles * Ts[0] // 4)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    act = sffn.TwellBuffers(cfg, Ts[0])
    for i, T in enumerate(Ts):
        print(f"[noalloc] {name} call {i} T={T}", flush=True)
        xs = x[:T].contiguous()
        y = torch.full_like(xs, float("nan"))
        layer.forward_noalloc(xs, act, y, workspace=(i == 1))
        assert sffn.check(act) == sffn.SFFN_OK
        y_ref, a_ref = layer.forward(xs)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (name, T)
        h, hr = act.to_host(), a_ref.to_host()
        for k in KEYS:
            assert np.array_equal(h[k].view(np.uint8), hr[k].view(np.uint8)), (name, T, k)
        assert h["bk_n"] == hr["bk_n"] and h["status"] == hr["status"] == 0


def test_noalloc_rejects_oversized_workspace():
    torch, sffn = need_gpu()
    c = CONFIGS["C3"]
    T = 8192
    # a backup capacity of every tile-row: the staged backup alone is 128 MiB
    cfg = _cfg(sffn, T, c, cap=c.n_tiles * T)
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    layer = sffn.SparseFFN(cfg, z(c.F, c.D), z(c.F), z(c.F, c.D))
    x = z(16, c.D)
    y = torch.empty_like(x)
    # 16 tokens fit (the staged backup is sized for the call's capacity: 16 * n_t entries)
    cfg16 = _cfg(sffn, 16, c, cap=c.n_tiles * 16)
    layer16 = sffn.SparseFFN(cfg16, z(c.F, c.D), z(c.F), z(c.F, c.D))
    act16 = sffn.TwellBuffers(cfg16, 16)
    layer16.forward_noalloc(x, act16, y)
    assert sffn.check(act16) == sffn.SFFN_OK
    assert not torch.any(y.float() != 0)
    big = sffn.TwellBuffers(cfg, 64)
    with pytest.raises(sffn.SffnError) as ei:
        layer.forward_noalloc(z(64, c.D), big, z(64, c.D))
    assert ei.value.status == sffn.SFFN_ERR_UNSUPPORTED
    assert "no-allocation scratch" in str(ei.value)
