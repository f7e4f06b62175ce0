"""The no-allocation entry point (ffn_swiglu_block_noalloc) against the
entry point it varies (ffn_swiglu_block with a caller workspace): the same
kernels on the same inputs give the same bits, call after call on the
library's one scratch array, the second call smaller than the first."""
import ctypes

import numpy as np
import pytest

from transformer_ffn_block_amd import inputs as I
from helpers import dev, host_bits

pytestmark = pytest.mark.gpu


def _abi_noalloc(L, ffn, dt, x, g, wg, wu, wd, y, eps, variant):
    M, d = x.shape
    f = wg.shape[0]
    return L.ffn_swiglu_block_noalloc(dt, x.data_ptr(), g.data_ptr(), wg.data_ptr(), wu.data_ptr(),
                                      wd.data_ptr(), y.data_ptr(), M, d, f, eps, ffn.VARIANTS[variant],
                                      None)


@pytest.mark.parametrize("variant,shapes", [
    ("auto", [(16, 1024, 2816), (3, 520, 712)]),          # decode kernels, then fewer tokens
    ("fused", [(300, 512, 768), (65, 256, 384)]),         # prefill GEMMs, then a smaller prefill
    ("split", [(64, 512, 704), (7, 264, 136)]),
    ("persistent", [(16, 1032, 384), (1, 64, 2056)]),
])
def test_noalloc_matches_workspace_entry_point(gpu_lib, variant, shapes):
    from transformer_ffn_block_amd import ffn
    import torch
    L = ffn.lib()
    for k, (M, d, f) in enumerate(shapes):
        print("noalloc", variant, M, d, f, flush=True)
        b = I.make_block(5000 + 10 * k + M, M, d, f, "bf16")
        x, g, wg, wu, wd = [dev(a) for a in (b.x, b.g, b.w_gate, b.w_up, b.w_down)]
        ref = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant=variant)
        y = torch.full_like(x, float("nan"))
        torch.cuda.synchronize()
        st = _abi_noalloc(L, ffn, ffn.FFN_BF16, x, g, wg, wu, wd, y, b.eps, variant)
        assert st == ffn.FFN_OK, L.ffn_last_error().decode()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), host_bits(ref)), (variant, M, d, f)


def test_noalloc_fp32_and_binding(gpu_lib):
    from transformer_ffn_block_amd import ffn
    import torch
    for M, d, f in ((8, 256, 704), (2, 36, 44)):
        b = I.make_block(5100 + M, M, d, f, "f32")
        x, g, wg, wu, wd = [dev(a, "f32") for a in (b.x, b.g, b.w_gate, b.w_up, b.w_down)]
        ref = ffn.swiglu_block(x, g, wg, wu, wd, b.eps)
        y = ffn.swiglu_block_noalloc(x, g, wg, wu, wd, b.eps)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


def test_noalloc_rejects_shapes_beyond_its_scratch(gpu_lib):
    from transformer_ffn_block_amd import ffn
    L = ffn.lib()
    M, d, f = 8192, 4096, 14336
    need = L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, M, d, f, ffn.VARIANTS["fused"])
    assert need > (16 << 20)
    # fake, never dereferenced addresses: the size check comes before any use
    st = L.ffn_swiglu_block_noalloc(ffn.FFN_BF16, 0x10000000, 0x20000000, 0x30000000, 0x40000000,
                                    0x50000000, 0x60000000, M, d, f, 1e-6, ffn.VARIANTS["fused"], None)
    assert st == ffn.FFN_ERR_UNSUPPORTED
    assert "scratch array holds 16777216" in L.ffn_last_error().decode()
