"""moe_layer_forward_noalloc (the library's fixed per-device scratch array in
place of a workspace) against moe_layer_forward on the same inputs: the same
kernels, so bitwise the same outputs, except for a Q8 shared expert on the
prefill path (dense GEMMs with a workspace, the grouped kernels without
one), where the outputs agree to the parity bar.  Two calls in a row, the
second with a smaller input (the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from quantized_moe_amd import lib, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _x(x, dt):
    if dt == synth.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def _both(dl, x, path):
    T = x.shape[0]
    out = []
    for noalloc in (False, True):
        y = torch.full((T, dl.d), float("nan"), dtype=torch.float32, device=DEV)
        idx = torch.full((T, dl.k), -1, dtype=torch.int32, device=DEV)
        wt = torch.full((T, dl.k), float("nan"), dtype=torch.float32, device=DEV)
        if noalloc:
            lib.layer_forward_noalloc(dl.desc, x, y, idx_out=idx, wt_out=wt, path=path)
        else:
            lib.layer_forward(dl.desc, x, y, dl.workspace(T), idx_out=idx, wt_out=wt, path=path)
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()))
    return out


REL_L2 = 1e-3


def _check(dl, x, path, bitwise=True):
    (y0, i0, w0), (y1, i1, w1) = _both(dl, x, path)
    assert np.all(np.isfinite(y0))
    assert np.array_equal(i1, i0)
    assert np.array_equal(w1, w0)
    if bitwise:
        assert np.array_equal(y1, y0)
    else:
        a, b = y1.astype(np.float64), y0.astype(np.float64)
        assert (np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)).max() <= REL_L2


def test_noalloc_full_size_decode_two_calls():
    """The 384-expert, top-6, d=4096, f=2048 layer: T = 24 (the automatic
    path's decode in three chunks of 8), then T = 8, then T = 1."""
    L = synth.random_layer(synth.DECODE_SPEC, seed=0, workload="decode")
    dl = lib.DeviceLayer.from_synth(L, DEV)
    try:
        for T in (24, 8, 1):
            x = _x(synth.activations(7, ("noalloc", "decode", T), T, 4096, synth.F32), synth.F32)
            _check(dl, x, lib.MOE_PATH_AUTO)
    finally:
        del dl
        torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt_shared", [synth.FMT_Q2K, synth.FMT_Q8])
def test_noalloc_small_layer_both_paths_two_calls(fmt_shared):
    """A small layer on the decode path (T = 6, then 2) and on the prefill
    path (T = 40, then 9) with bf16 x, a router bias and down gains; with a
    Q8 shared expert the prefill outputs agree to the parity bar."""
    spec = synth.scaled_spec(E=32, k=4, d=1024, f=512, fmt_shared=fmt_shared)
    L = synth.random_layer(spec, seed=8, workload="noalloc")
    rng = np.random.default_rng(8)
    L = synth.Layer(**{**L.__dict__, "router_bias": rng.normal(0, 0.05, spec.E).astype(np.float32),
                       "down_gain": rng.uniform(0.5, 1.5, (spec.E, spec.d)).astype(np.float32)})
    dl = lib.DeviceLayer.from_synth(L, DEV)
    for path, Ts in ((lib.MOE_PATH_DECODE, (6, 2)), (lib.MOE_PATH_PREFILL, (40, 9))):
        for T in Ts:
            x = _x(synth.activations(8, ("noalloc", path, T), T, spec.d, synth.BF16), synth.BF16)
            _check(dl, x, path, bitwise=path == lib.MOE_PATH_DECODE or fmt_shared != synth.FMT_Q8)


def test_noalloc_rejects_calls_above_its_scratch():
    """A 1024-token prefill chunk of the full layer needs ~150 MB of
    workspace: refused before anything is enqueued, with a clear message."""
    spec = synth.DECODE_SPEC
    L = synth.random_layer(synth.scaled_spec(E=8, k=spec.k, d=spec.d, f=spec.f), seed=1, workload="noalloc-big")
    dl = lib.DeviceLayer.from_synth(L, DEV)
    T = 1024
    assert lib.workspace_bytes(dl.desc, T, lib.MOE_OP_LAYER) > lib.MOE_NOALLOC_SCRATCH_BYTES
    x = _x(synth.activations(9, ("noalloc", "big"), T, spec.d, synth.BF16), synth.BF16)
    y = torch.zeros(T, spec.d, dtype=torch.float32, device=DEV)
    with pytest.raises(lib.MoeError) as ei:
        lib.layer_forward_noalloc(dl.desc, x, y)
    assert ei.value.status == lib.MOE_ERR_WORKSPACE
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0  # nothing ran
