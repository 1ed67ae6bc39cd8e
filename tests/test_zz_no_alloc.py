"""moe_forward_static, the forward for callers that cannot allocate (HIP graph
capture, serving loops, harnesses without hipMalloc), against moe_forward with a
caller workspace: the same kernels on the same inputs, so every output must be
bit-identical.  Two calls in a row share the library's buffer, the second with
fewer tokens (and the caller's workspace filled with garbage first)."""
import numpy as np
import pytest

import moe_synth as syn
from _util import shape_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_35_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _cfg(dtype, Ns=1):
    return syn.LayerConfig("noalloc", T=300, d=256, Nr=16, G=4, Mg=2, K=3, Ns=Ns, I=256, dtype=dtype,
                           bias="uniform")


def _outputs(moe, cfg, T, static, layer, u, flags=0):
    shape = shape_of(cfg, T=T, flags=flags)
    dt = u.dtype
    out = torch.full((T, cfg.d), 7.0, dtype=dt, device="cuda")
    idx = torch.full((T, cfg.K), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, cfg.K), -1.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((cfg.Nr,), -1, dtype=torch.int32, device="cuda")
    sc = torch.full((T, cfg.Nr), -1.0, dtype=torch.float32, device="cuda")
    args = (shape, u[:T], layer.gate_w, layer.bias, layer.routed_w, layer.routed_s, layer.shared_w, layer.shared_s,
            out, idx, w, cnt, sc)
    if static:
        moe.moe_forward_static(*args)
    else:
        ws = torch.empty(moe.moe_workspace_bytes(shape, moe.MOE_WS_FORWARD), dtype=torch.uint8, device="cuda")
        ws.fill_(0xA5)
        moe.moe_forward(*args, ws=ws)
    torch.cuda.synchronize()
    return [t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
            for t in (out, idx, w, cnt, sc)]


@pytest.mark.parametrize("dtype,Ns,flags", [("fp32", 1, 0), ("bf16", 1, 1), ("fp8", 2, 0), ("bf16", 0, 0)])
def test_static_forward_equals_forward_twice(moe, dtype, Ns, flags):
    from mixture_experts_layer_35_amd.layer import MoeLayer, to_device
    cfg = _cfg(dtype, Ns)
    inp = syn.layer_inputs(cfg, seed=31)
    layer = MoeLayer.from_host(shape_of(cfg), inp["gate_w"], inp["bias"], inp["wg"], inp["wu"], inp["wd"],
                               inp["swg"], inp["swu"], inp["swd"])
    u = to_device(inp["u"])
    for T in (cfg.T, 77):          # the second call is smaller and reuses the library's buffer
        print("moe_forward_static", dtype, "Ns", Ns, "flags", flags, "T", T, flush=True)
        got = _outputs(moe, cfg, T, True, layer, u, flags)
        ref = _outputs(moe, cfg, T, False, layer, u, flags)
        for g, r, name in zip(got, ref, ("out", "topk_idx", "topk_w", "counts", "scores")):
            assert g.shape == r.shape, name
            assert (g.view(np.uint8) == r.view(np.uint8)).all(), (name, T)
        assert (got[1] >= 0).all() and got[3].sum() == T * cfg.K


def test_static_forward_rejects_what_does_not_fit(moe):
    cfg = syn.CONFIGS["v3_prefill"]
    shape = shape_of(cfg)
    assert moe.moe_workspace_bytes(shape, moe.MOE_WS_FORWARD) > moe.MOE_STATIC_WS_BYTES
    fake = 1 << 20
    w3 = (fake, fake, fake)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_static(shape, fake, fake, fake, w3, None, w3, None, fake)
    assert e.value.code == moe.MOE_ERR_WORKSPACE
    small = shape_of(_cfg("bf16"), flags=moe.MOE_SAVE_SWIGLU_INPUTS)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_static(small, fake, fake, fake, w3, None, w3, None, fake)
    assert e.value.code == moe.MOE_ERR_UNSUPPORTED
