"""The Python binding's own argument checks, on the CPU: every rule raises
TypeError / ValueError before any device work.  The tensors here are CPU
tensors; the binding checks dtypes, layouts and shapes first and the device
last, so each rule is reached on its own, and a call whose tensors are right
in every other way fails at the device check ("How to Use FlashKDA as a
Backend for flash-linear-attention", "Kernel API and Tensor Requirements":
bf16 q/k/v/g/beta, fp32 A_log/dt_bias, lower_bound range, state shapes; the
cuLA PR #106 review thread: errors instead of implicit conversions, CPU
tensors rejected)."""
import pytest

torch = pytest.importorskip("torch")

import kimi_delta_attention_02_amd as kda  # noqa: E402

B, T, H, D = 1, 32, 2, 128


def _tensors(**over):
    bf = torch.bfloat16
    t = dict(
        q=torch.zeros(B, T, H, D, dtype=bf), k=torch.zeros(B, T, H, D, dtype=bf), v=torch.zeros(B, T, H, D, dtype=bf),
        g=torch.zeros(B, T, H, D, dtype=bf), beta=torch.zeros(B, T, H, dtype=bf),
        A_log=torch.zeros(H, dtype=torch.float32), dt_bias=torch.zeros(H, D, dtype=torch.float32),
        initial_state=None, final_state=None, cu_seqlens=None, out=None, workspace=None)
    t.update(over)
    return t


def _fwd(**over):
    t = _tensors(**over)
    extra = {k: t.pop(k) for k in ("state_layout", "cp_mode") if k in t}
    return kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], 0.1, t["out"], A_log=t["A_log"], dt_bias=t["dt_bias"],
                   lower_bound=-1.0, workspace=t["workspace"], initial_state=t["initial_state"],
                   final_state=t["final_state"], cu_seqlens=t["cu_seqlens"], **extra)


bf16 = torch.bfloat16
f32 = torch.float32

CASES = [
    # non-tensors and wrong dtypes: no implicit conversion
    (dict(q=[[0.0]]), TypeError, "q must be a torch.Tensor"),
    (dict(q=torch.zeros(B, T, H, D, dtype=f32)), TypeError, "q must be torch.bfloat16"),
    (dict(k=torch.zeros(B, T, H, D, dtype=torch.float16)), TypeError, "k must be torch.bfloat16"),
    (dict(v=torch.zeros(B, T, H, D, dtype=f32)), TypeError, "v must be torch.bfloat16"),
    (dict(g=torch.zeros(B, T, H, D, dtype=f32)), TypeError, "g must be torch.bfloat16"),
    (dict(beta=torch.zeros(B, T, H, dtype=f32)), TypeError, "beta must be torch.bfloat16"),
    (dict(A_log=torch.zeros(H, dtype=torch.float64)), TypeError, "A_log must be torch.float32"),
    (dict(dt_bias=torch.zeros(H, D, dtype=bf16)), TypeError, "dt_bias must be torch.float32"),
    (dict(cu_seqlens=torch.tensor([0, T], dtype=torch.int64)), TypeError, "cu_seqlens must be torch.int32"),
    (dict(initial_state=torch.zeros(1, H, D, D, dtype=torch.float16)), TypeError, "float32 or bfloat16"),
    (dict(final_state="state"), TypeError, "final_state must be a torch.Tensor"),
    (dict(initial_state=torch.zeros(1, H, D, D, dtype=f32), final_state=torch.zeros(1, H, D, D, dtype=bf16)),
     TypeError, "same dtype"),
    (dict(out=torch.zeros(B, T, H, D, dtype=f32)), TypeError, "out must be torch.bfloat16"),
    (dict(workspace=torch.zeros(1024, dtype=f32)), TypeError, "workspace must be torch.uint8"),
    # layouts
    (dict(q=torch.zeros(B, T, D, H, dtype=bf16).transpose(2, 3)), ValueError, "q must be contiguous"),
    (dict(k=torch.zeros(B, H, T, D, dtype=bf16).transpose(1, 2)), ValueError, "k must be contiguous"),
    (dict(initial_state=torch.zeros(1, H, D, D, dtype=f32).transpose(2, 3)), ValueError,
     "initial_state must be contiguous"),
    # shapes
    (dict(q=torch.zeros(B, T, H * D, dtype=bf16)), ValueError, "must be [B, T, heads, D]"),
    (dict(q=torch.zeros(B, T, H, 64, dtype=bf16), k=torch.zeros(B, T, H, 64, dtype=bf16),
          v=torch.zeros(B, T, H, 64, dtype=bf16)), ValueError, "head dimension must be 128"),
    (dict(v=torch.zeros(B, T, 3, D, dtype=bf16)), ValueError, "multiple of q's"),
    (dict(v=torch.zeros(B, T + 1, H, D, dtype=bf16)), ValueError, "expected [B, T, H, D]"),
    (dict(k=torch.zeros(B, T, 1, D, dtype=bf16)), ValueError, "k has shape"),
    (dict(g=torch.zeros(B, T, H, D + 2, dtype=bf16)), ValueError, "g has shape"),
    (dict(beta=torch.zeros(B, T, dtype=bf16)), ValueError, "beta has shape"),
    (dict(A_log=torch.zeros(H + 1, dtype=f32)), ValueError, "A_log has shape"),
    (dict(dt_bias=torch.zeros(H, dtype=f32)), ValueError, "dt_bias has shape"),
    (dict(out=torch.zeros(B, T, H, 64, dtype=bf16)), ValueError, "out has shape"),
    (dict(initial_state=torch.zeros(2, H, D, D, dtype=f32)), ValueError, "initial_state has shape"),
    (dict(final_state=torch.zeros(1, H, D, D // 2, dtype=bf16)), ValueError, "final_state has shape"),
    # varlen rules: int32 offsets, 1-D, at least two entries, B == 1
    (dict(cu_seqlens=torch.tensor([[0, T]], dtype=torch.int32)), ValueError, "cu_seqlens must be 1-D"),
    (dict(cu_seqlens=torch.tensor([0], dtype=torch.int32)), ValueError, "cu_seqlens must be 1-D"),
    (dict(q=torch.zeros(2, T, H, D, dtype=bf16), k=torch.zeros(2, T, H, D, dtype=bf16),
          v=torch.zeros(2, T, H, D, dtype=bf16), g=torch.zeros(2, T, H, D, dtype=bf16),
          beta=torch.zeros(2, T, H, dtype=bf16), cu_seqlens=torch.tensor([0, 10, 2 * T], dtype=torch.int32)),
     ValueError, "cu_seqlens requires B == 1"),
    (dict(cu_seqlens=torch.tensor([0, 10, T], dtype=torch.int32), initial_state=torch.zeros(1, H, D, D, dtype=f32)),
     ValueError, "initial_state has shape"),
    # other arguments
    (dict(state_layout="xy"), ValueError, "state_layout must be"),
    (dict(cp_mode="sometimes"), ValueError, "cp_mode must be"),
    (dict(cp_mode=7), ValueError, "cp_mode must be"),
    # right in every way but on the CPU
    (dict(), ValueError, "q must be a GPU tensor"),
    (dict(initial_state=torch.zeros(1, H, D, D, dtype=f32)), ValueError, "must be a GPU tensor"),
]


@pytest.mark.parametrize("over,exc,msg", CASES, ids=[c[2] for c in CASES])
def test_fwd_argument_checks(over, exc, msg):
    with pytest.raises(exc) as ei:
        _fwd(**over)
    assert msg in str(ei.value)


def test_noalloc_needs_out_and_applies_the_same_checks():
    t = _tensors()
    with pytest.raises(ValueError, match="needs out"):
        kda.fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], 0.1, None, A_log=t["A_log"], dt_bias=t["dt_bias"],
                        lower_bound=-1.0)
    with pytest.raises(TypeError, match="beta must be torch.bfloat16"):
        kda.fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"].float(), 0.1, torch.zeros_like(t["q"]),
                        A_log=t["A_log"], dt_bias=t["dt_bias"], lower_bound=-1.0)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], 0.1, torch.zeros_like(t["q"]), A_log=t["A_log"],
                        dt_bias=t["dt_bias"], lower_bound=-1.0)


def test_prepare_applies_the_same_checks():
    t = _tensors()
    with pytest.raises(TypeError, match="dt_bias must be torch.float32"):
        kda.prepare(t["q"], t["k"], t["v"], t["g"], t["beta"], 0.1, A_log=t["A_log"], dt_bias=t["dt_bias"].double(),
                    lower_bound=-1.0)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.prepare(t["q"], t["k"], t["v"], t["g"], t["beta"], 0.1, A_log=t["A_log"], dt_bias=t["dt_bias"],
                    lower_bound=-1.0)


def test_chunk_kda_checks_before_device_work():
    t = _tensors()
    with pytest.raises(TypeError, match="q must be torch.bfloat16"):
        kda.chunk_kda(t["q"].float(), t["k"], t["v"], t["g"], t["beta"], A_log=t["A_log"], dt_bias=t["dt_bias"],
                      lower_bound=-1.0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        kda.chunk_kda(t["q"], t["k"], t["v"], t["g"], t["beta"], A_log=t["A_log"], dt_bias=t["dt_bias"],
                      lower_bound=-1.0)
