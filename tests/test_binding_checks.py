"""The Python binding checks every tensor argument before its pointer reaches the
library (CPU only).

The C ABI can check only what a pointer carries: NULL, alignment and overlap.
A wrong dtype, shape, contiguity or device of an output or of lse must
therefore be refused by the binding itself, with ValueError (TypeError for a
non-tensor or for q, k, v of the wrong format), before anything is allocated
or launched.  The checks run here on CPU tensors (``require_gpu=False``); a
``meta`` tensor stands in for a tensor on another device.
"""
import os

import pytest
import torch

from exact_io_aware_26_amd import fa2

B, Hq, Hkv, N, d = 2, 4, 2, 10, 64


def qkv(dtype=torch.bfloat16):
    return (torch.zeros(B, Hq, N, d, dtype=dtype), torch.zeros(B, Hkv, N, d, dtype=dtype),
            torch.zeros(B, Hkv, N, d, dtype=dtype))


def test_forward_args_accepted():
    q, k, v = qkv()
    out, lse = torch.empty_like(q), torch.empty(B, Hq, N)
    assert fa2.check_forward_args(q, k, v, out, lse, require_gpu=False) == (B, Hq, Hkv, N, d)


@pytest.mark.parametrize("bad", ["dtype", "shape", "noncontig", "device"])
def test_forward_lse_and_out_checked(bad):
    q, k, v = qkv()
    lse = {"dtype": torch.empty(B, Hq, N, dtype=torch.float64),
           "shape": torch.empty(B, Hq, N - 1),
           "noncontig": torch.empty(B, N, Hq).transpose(1, 2),
           "device": torch.empty(B, Hq, N, device="meta")}[bad]
    with pytest.raises(ValueError, match="lse"):
        fa2.check_forward_args(q, k, v, None, lse, require_gpu=False)
    out = {"dtype": torch.empty(B, Hq, N, d, dtype=torch.float16),
           "shape": torch.empty(B, Hq, N, d + 1, dtype=torch.bfloat16),
           "noncontig": torch.empty(B, Hq, d, N, dtype=torch.bfloat16).transpose(2, 3),
           "device": torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device="meta")}[bad]
    with pytest.raises(ValueError, match="out"):
        fa2.check_forward_args(q, k, v, out, None, require_gpu=False)


def test_inputs_checked():
    q, k, v = qkv()
    with pytest.raises(TypeError):
        fa2.check_forward_args(q.float(), k, v, require_gpu=False)
    with pytest.raises(TypeError):
        fa2.check_forward_args(q, k.half(), v, require_gpu=False)
    with pytest.raises(ValueError, match="device"):
        fa2.check_forward_args(q, k.to("meta"), v, require_gpu=False)
    with pytest.raises(ValueError, match="shape mismatch"):
        fa2.check_forward_args(q, k[:, :, :-1].contiguous(), v, require_gpu=False)
    with pytest.raises(ValueError, match="GPU"):
        fa2.check_forward_args(q, k, v)          # CPU tensors on the real entry points


def test_backward_args_checked():
    q, k, v = qkv()
    o, do, lse = torch.empty_like(q), torch.empty_like(q), torch.empty(B, Hq, N)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(4096, dtype=torch.uint8)
    ok = dict(workspace=ws, grads=grads, nbytes=4096, require_gpu=False)
    assert fa2.check_backward_args(q, k, v, o, lse, do, **ok) == (B, Hq, Hkv, N, d)
    cases = {
        "o": lambda a: a.update(o=o[..., :-1]),
        "do": lambda a: a.update(do=do.float()),
        "lse": lambda a: a.update(lse=lse.to("meta")),
        "workspace": lambda a: a.update(workspace=ws[:100]),
        "dk": lambda a: a.update(grads=(grads[0], grads[2][:, :1], grads[2])),
        "dq": lambda a: a.update(grads=(grads[0].to("meta"), grads[1], grads[2])),
    }
    for name, mutate in cases.items():
        args = dict(o=o, lse=lse, do=do)
        mutate(args)
        with pytest.raises(ValueError, match=name):
            fa2.check_backward_args(q, k, v, args["o"], args["lse"], args["do"],
                                    workspace=ws if name != "workspace" else args.get("workspace"),
                                    grads=args.get("grads", grads), nbytes=4096, require_gpu=False)
    with pytest.raises(ValueError, match="workspace"):
        fa2.check_backward_args(q, k, v, o, lse, do, workspace=ws.view(64, 64), nbytes=16,
                                require_gpu=False)


@pytest.mark.skipif(not os.path.exists(fa2.LIB_PATH), reason="libfa2.so not built")
def test_entry_points_refuse_cpu_tensors_before_any_launch():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="GPU"):
        fa2.forward(q, k, v)
    o, do, lse = torch.empty_like(q), torch.empty_like(q), torch.empty(B, Hq, N)
    with pytest.raises(ValueError, match="GPU"):
        fa2.backward(q, k, v, o, lse, do)
    with pytest.raises(ValueError, match="GPU"):
        fa2.forward_block_sparse(q, k, v, torch.ones(1, 1, dtype=torch.uint8))


@pytest.mark.parametrize("bad", ["dtype", "shape", "noncontig", "device"])
def test_o_lo_checked(bad):
    """The split-O residual: a bf16 tensor shaped like q on q's device, for bf16 calls only."""
    q, k, v = qkv()
    o_lo = {"dtype": torch.empty(B, Hq, N, d, dtype=torch.float16),
            "shape": torch.empty(B, Hq, N, d - 8, dtype=torch.bfloat16),
            "noncontig": torch.empty(B, Hq, d, N, dtype=torch.bfloat16).transpose(2, 3),
            "device": torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device="meta")}[bad]
    with pytest.raises(ValueError, match="o_lo"):
        fa2.check_forward_args(q, k, v, None, None, require_gpu=False, o_lo=o_lo)
    o, do, lse = torch.empty_like(q), torch.empty_like(q), torch.empty(B, Hq, N)
    with pytest.raises(ValueError, match="o_lo"):
        fa2.check_backward_args(q, k, v, o, lse, do, require_gpu=False, o_lo=o_lo)
    q16, k16, v16 = qkv(torch.float16)
    with pytest.raises(TypeError, match="o_lo"):
        fa2.check_forward_args(q16, k16, v16, require_gpu=False, o_lo=torch.empty_like(q16))
    fa2.check_forward_args(q, k, v, require_gpu=False, o_lo=torch.empty_like(q))
