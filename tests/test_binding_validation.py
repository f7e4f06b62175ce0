"""The Python binding checks every operand against (M, d, f) before it hands
a raw pointer to the library: wrong shapes, dtypes, layouts, devices,
workspaces and quantised-weight pairs raise ValueError (or FFNError for a
short workspace) without any launch.  CPU only: the tensors are host
tensors, so a call that got past the checks would stop at the first device
pointer ("must be a device tensor"), never at a kernel."""
import pytest
import torch

from transformer_ffn_block_amd import ffn

BF = torch.bfloat16
M, d, f = 4, 64, 96


def _block(**over):
    t = dict(x=torch.zeros(M, d, dtype=BF), g=torch.zeros(d, dtype=BF),
             w_gate=torch.zeros(f, d, dtype=BF), w_up=torch.zeros(f, d, dtype=BF),
             w_down=torch.zeros(d, f, dtype=BF))
    t.update(over)
    return t


def _call(**over):
    t = _block(**over)
    extra = {k: t.pop(k) for k in ("out", "workspace", "variant") if k in t}
    return ffn.swiglu_block(t["x"], t["g"], t["w_gate"], t["w_up"], t["w_down"], 1e-6, **extra)


@pytest.mark.parametrize("over,msg", [
    (dict(w_up=torch.zeros(f + 8, d, dtype=BF)), "w_up has shape"),
    (dict(w_down=torch.zeros(f, d, dtype=BF)), "w_down has shape"),     # transposed down weights
    (dict(w_gate=torch.zeros(f, d + 8, dtype=BF)), "w_gate has shape"),
    (dict(g=torch.zeros(d + 8, dtype=BF)), "g has shape"),
    (dict(g=torch.zeros(d, dtype=torch.float32)), "g has dtype"),
    (dict(w_down=torch.zeros(d, f, dtype=torch.float32)), "w_down has dtype"),
    (dict(x=torch.zeros(M, d, 1, dtype=BF)), "2-D"),
    (dict(w_up=torch.zeros(d, f, dtype=BF).t()), "must be contiguous"),
    (dict(out=torch.zeros(M, d + 8, dtype=BF)), "out has shape"),
    (dict(out=torch.zeros(M, d, dtype=torch.float32)), "out has dtype"),
    (dict(variant="fastest"), "unknown variant"),
    (dict(w_gate=torch.zeros(f, d, dtype=BF, device="meta")), "w_gate is on meta"),
])
def test_block_rejects_mismatched_operands(over, msg):
    with pytest.raises(ValueError, match=msg):
        _call(**over)


def test_block_rejects_small_or_foreign_workspace():
    with pytest.raises(ffn.FFNError, match="needed"):
        _call(workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace is on meta"):
        _call(workspace=torch.zeros(1 << 20, dtype=torch.uint8, device="meta"))


def test_block_with_consistent_host_tensors_stops_at_the_device_check():
    with pytest.raises(ValueError, match="must be a device tensor"):
        _call()


def test_rmsnorm_rejects_mismatched_gain():
    with pytest.raises(ValueError, match="g has shape"):
        ffn.rmsnorm(torch.zeros(3, 64, dtype=BF), torch.zeros(72, dtype=BF), 1e-6)
    with pytest.raises(ValueError, match="g has dtype"):
        ffn.rmsnorm(torch.zeros(3, 64, dtype=BF), torch.zeros(64, dtype=torch.float32), 1e-6)
    with pytest.raises(TypeError, match="unsupported dtype"):
        ffn.rmsnorm(torch.zeros(3, 64, dtype=torch.float16), torch.zeros(64, dtype=torch.float16), 1e-6)


def _q8(N, K):
    return torch.zeros(N, K, dtype=torch.int8), torch.zeros(N, K // 32, dtype=torch.int16)


def _q4(N, K):
    return torch.zeros(N, K // 2, dtype=torch.uint8), torch.zeros(N, K // 32, dtype=torch.int16)


@pytest.mark.parametrize("kind", ["q8", "q4"])
def test_quant_block_rejects_mismatched_pairs(kind):
    mk = _q8 if kind == "q8" else _q4
    fn = ffn.swiglu_block_q8 if kind == "q8" else ffn.swiglu_block_q4
    x, g = torch.zeros(M, d, dtype=BF), torch.zeros(d, dtype=BF)
    good = dict(w_gate=mk(f, d), w_up=mk(f, d), w_down=mk(d, f))

    def call(**over):
        w = dict(good, **over)
        return fn(over.pop("x", x), g, w["w_gate"], w["w_up"], w["w_down"], 1e-6)

    with pytest.raises(ValueError, match="w_down quants has shape"):
        call(w_down=mk(f, d))                                  # transposed
    with pytest.raises(ValueError, match="w_up scales has shape"):
        call(w_up=(mk(f, d)[0], torch.zeros(f, d // 16, dtype=torch.int16)))
    with pytest.raises(ValueError, match="quants has dtype"):
        other = torch.uint8 if kind == "q8" else torch.int8
        call(w_gate=(mk(f, d)[0].to(other), mk(f, d)[1]))
    with pytest.raises(ValueError, match="scales has dtype"):
        call(w_gate=(mk(f, d)[0], torch.zeros(f, d // 32, dtype=torch.float16)))
    with pytest.raises(ValueError, match="pair"):
        call(w_up=mk(f, d)[0])
    with pytest.raises(ValueError, match="x has dtype"):
        fn(torch.zeros(M, d, dtype=torch.float32), g, good["w_gate"], good["w_up"], good["w_down"], 1e-6)
    with pytest.raises(ValueError, match="must be a device tensor"):
        call()


def test_prepared_quant_call_checks_its_operands():
    x, g = torch.zeros(M, d, dtype=BF), torch.zeros(d, dtype=BF)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="kind"):
        ffn.prepare_swiglu_block_quant("q5", x, g, _q8(f, d), _q8(f, d), _q8(d, f), 1e-6, x.clone(), ws)
    with pytest.raises(ValueError, match="w_down quants has shape"):
        ffn.prepare_swiglu_block_quant("q8", x, g, _q8(f, d), _q8(f, d), _q8(f, d), 1e-6, x.clone(), ws)
    with pytest.raises(ffn.FFNError, match="needed"):
        ffn.prepare_swiglu_block_quant("q8", x, g, _q8(f, d), _q8(f, d), _q8(d, f), 1e-6, x.clone(),
                                       torch.zeros(16, dtype=torch.uint8))
