"""The Python binding rejects caller-supplied output buffers that the kernels
would write past or misread (CPU only: the checks run before any launch)."""
import pytest
import torch

from tiled_attention_13_amd._binding import _check_out


def test_matching_output_is_accepted():
    _check_out("out", torch.empty((1, 2, 3, 32), dtype=torch.bfloat16), (1, 2, 3, 32), torch.bfloat16,
               torch.device("cpu"))


@pytest.mark.parametrize("bad,what", [
    (lambda: torch.empty((1, 2, 3, 16), dtype=torch.bfloat16), "shape"),        # too small
    (lambda: torch.empty((1, 2, 4, 32), dtype=torch.bfloat16), "shape"),        # too large is still wrong
    (lambda: torch.empty((1, 2, 3, 32), dtype=torch.float32), "dtype"),         # f32 buffer for a bf16 output
    (lambda: torch.empty((1, 2, 32, 3), dtype=torch.bfloat16).transpose(2, 3), "contiguous"),
    (lambda: torch.empty((1, 2, 3, 32), dtype=torch.bfloat16, device="meta"), "must be on"),
])
def test_bad_output_is_rejected(bad, what):
    with pytest.raises(ValueError, match=what):
        _check_out("out", bad(), (1, 2, 3, 32), torch.bfloat16, torch.device("cpu"))


def test_lse_must_be_float32():
    with pytest.raises(ValueError, match="dtype"):
        _check_out("lse", torch.empty((1, 2, 3), dtype=torch.bfloat16), (1, 2, 3), torch.float32,
                   torch.device("cpu"))


@pytest.mark.gpu
def test_entry_points_reject_bad_outputs(gpu_lib):
    """Every wrapper that takes an output buffer refuses a wrong one before launching."""
    import tiled_attention_13_amd as fa
    dev = "cuda"
    q, k, v = (torch.randn((1, 2, 100, 64), device=dev).to(torch.bfloat16) for _ in range(3))
    short = torch.empty((1, 2, 99, 64), dtype=torch.bfloat16, device=dev)
    f32 = torch.empty((1, 2, 100, 64), dtype=torch.float32, device=dev)
    lse_bad = torch.empty((1, 2, 99), dtype=torch.float32, device=dev)
    o, lse = fa.fwd(q, k, v, causal=True)
    mask = torch.ones((2, 2), dtype=torch.uint8, device=dev)
    parts_o = torch.zeros((2, 1, 2, 100, 64), dtype=torch.float32, device=dev)
    parts_l = torch.zeros((2, 1, 2, 100), dtype=torch.float32, device=dev)
    calls = [
        lambda: fa.fwd(q, k, v, out=short),
        lambda: fa.fwd(q, k, v, out=f32),
        lambda: fa.fwd(q, k, v, lse=lse_bad),
        lambda: fa.fwd_splitkv(q, k, v, 2, out=short),
        lambda: fa.fwd_blocksparse(q, k, v, mask, lse=lse_bad),
        lambda: fa.fwd_partial(q, k, v, 0, 64, o_part=o),
        lambda: fa.merge(parts_o, parts_l, out=f32),
        lambda: fa.merge(parts_o, parts_l.cpu()),
        lambda: fa.bwd(q, k, v, o, o, lse, dq=short),
        lambda: fa.bwd(q, k, v, o, o, lse, dv=f32),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
