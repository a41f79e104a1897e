"""The Python binding rejects output, scale and work buffers that do not match
what the kernels write, before any launch. Runs without a GPU: the inputs are
stand-ins that report a GPU device (the binding reads only their shape, type,
device, layout and address), and any call that got past the checks would fail
at the stream lookup with a different error, never with ValueError."""
import pytest
import torch

import io_aware_softmax_fa_amd as fa

GPU = torch.device("cuda:0")


class Dev:
    """A CPU tensor that reports a GPU device."""

    def __init__(self, t, device=GPU):
        self.t, self.device = t, device

    shape = property(lambda self: self.t.shape)
    dtype = property(lambda self: self.t.dtype)

    def dim(self):
        return self.t.dim()

    def is_contiguous(self):
        return self.t.is_contiguous()

    def numel(self):
        return self.t.numel()

    def element_size(self):
        return self.t.element_size()

    def data_ptr(self):
        return self.t.data_ptr()

    def transpose(self, a, b):
        return Dev(self.t.transpose(a, b), self.device)


def dev(shape, dtype=torch.bfloat16, device=GPU):
    return Dev(torch.zeros(shape, dtype=dtype), device)


QS = (1, 2, 64, 128)


def _bad_outputs(shape, dtype):
    """Output tensors that differ from (shape, dtype, GPU, contiguous) in one way."""
    n = len(shape)
    short = tuple(shape[:-1]) + (shape[-1] - 1,)
    yield "short", dev(short, dtype)
    yield "dtype", dev(shape, torch.float32 if dtype != torch.float32 else torch.float16)
    yield "host", Dev(torch.zeros(shape, dtype=dtype), torch.device("cpu"))
    if n >= 2 and shape[-1] > 1 and shape[-2] > 1:
        t = torch.zeros(tuple(shape[:-2]) + (shape[-1], shape[-2]), dtype=dtype).transpose(-1, -2)
        yield "strided", Dev(t)


@pytest.mark.parametrize("which", ["out", "lse"])
def test_forward_rejects_bad_outputs(which):
    q = dev(QS)
    good = {"out": dev(QS), "lse": dev(QS[:3], torch.float32)}
    shape, dtype = (QS, torch.bfloat16) if which == "out" else (QS[:3], torch.float32)
    for why, bad in _bad_outputs(shape, dtype):
        kw = dict(good, **{which: bad})
        with pytest.raises(ValueError):
            fa.forward(q, q, q, **kw)


def test_forward_fp8_rejects_bad_outputs_and_host_inputs():
    q8 = dev(QS, torch.uint8)
    good = {"out": dev(QS), "lse": dev(QS[:3], torch.float32)}
    for which, shape, dtype in (("out", QS, torch.bfloat16), ("lse", QS[:3], torch.float32)):
        for why, bad in _bad_outputs(shape, dtype):
            with pytest.raises(ValueError):
                fa.forward_fp8(q8, q8, q8, (1.0, 1.0, 1.0), **dict(good, **{which: bad}))
    host = Dev(torch.zeros(QS, dtype=torch.uint8), torch.device("cpu"))
    with pytest.raises(ValueError):
        fa.forward_fp8(host, host, host, (1.0, 1.0, 1.0), **good)


def test_forward_fp8_block_rejects_bad_scales_and_outputs():
    B, H, N, d = QS
    q8 = dev(QS, torch.uint8)
    scales = [dev((B, H, -(-N // r)), torch.float32) for r in (128, 64, 64)]
    good = {"out": dev(QS), "lse": dev(QS[:3], torch.float32)}
    host_scale = Dev(torch.zeros((B, H, 1)), torch.device("cpu"))
    with pytest.raises(ValueError):
        fa.forward_fp8_block(q8, q8, q8, host_scale, scales[1], scales[2], **good)
    with pytest.raises(ValueError):
        fa.forward_fp8_block(q8, q8, q8, scales[0], dev((B, H, 2), torch.float32), scales[2], **good)
    for which, shape, dtype in (("out", QS, torch.bfloat16), ("lse", QS[:3], torch.float32)):
        for why, bad in _bad_outputs(shape, dtype):
            with pytest.raises(ValueError):
                fa.forward_fp8_block(q8, q8, q8, *scales, **dict(good, **{which: bad}))


@pytest.mark.parametrize("which", ["dq", "dk", "dv", "workspace"])
def test_backward_rejects_bad_buffers(which):
    q = dev(QS)
    lse = dev(QS[:3], torch.float32)
    B, H, N, d = QS
    good = {"dq": dev(QS), "dk": dev(QS), "dv": dev(QS),
            "workspace": dev((2 * B * H * N,), torch.float32)}
    if which == "workspace":
        bads = [dev((2 * B * H * N - 1,), torch.float32), dev((2 * B * H * N,), torch.float16),
                Dev(torch.zeros(2 * B * H * N), torch.device("cpu"))]
    else:
        bads = [b for _, b in _bad_outputs(QS, torch.bfloat16)]
    for bad in bads:
        with pytest.raises(ValueError):
            fa.backward(q, q, q, q, lse, q, **dict(good, **{which: bad}))


def test_forward_kv_rejects_bad_buffers():
    B, H, Hkv, Nq, Nk, d = 1, 4, 2, 8, 256, 128
    q = dev((B, H, Nq, d))
    kv = dev((B, Hkv, Nk, d))
    good = {"out": dev((B, H, Nq, d)), "lse": dev((B, H, Nq), torch.float32)}
    for which, shape, dtype in (("out", (B, H, Nq, d), torch.bfloat16),
                                ("lse", (B, H, Nq), torch.float32)):
        for why, bad in _bad_outputs(shape, dtype):
            with pytest.raises(ValueError):
                fa.forward_kv(q, kv, kv, num_splits=1, **dict(good, **{which: bad}))
    need = fa.fa_fwd_kv_workspace(B, H, Nq, d, 4)
    for bad in (dev((need // 4 - 1,), torch.float32),
                Dev(torch.zeros(need // 4), torch.device("cpu"))):
        with pytest.raises(ValueError):
            fa.forward_kv(q, kv, kv, num_splits=4, workspace=bad, **good)


def test_forward_varlen_rejects_bad_buffers():
    total, H, Hkv, d = 100, 4, 2, 64
    q = dev((total, H, d), torch.float16)
    kv = dev((total, Hkv, d), torch.float16)
    cu = dev((3,), torch.int32)
    good = {"out": dev((total, H, d), torch.float16), "lse": dev((total, H), torch.float32)}
    for which, shape, dtype in (("out", (total, H, d), torch.float16),
                                ("lse", (total, H), torch.float32)):
        for why, bad in _bad_outputs(shape, dtype):
            with pytest.raises(ValueError):
                fa.forward_varlen(q, kv, kv, cu, cu, 60, 60, **dict(good, **{which: bad}))
    need = fa.fa_fwd_varlen_workspace(total, H, d, 2)
    with pytest.raises(ValueError):
        fa.forward_varlen(q, kv, kv, cu, cu, 60, 60, num_splits=2,
                          workspace=dev((need // 4 - 1,), torch.float32), **good)


def test_quantize_rejects_bad_outputs():
    x = dev((1, 2, 100, 64), torch.float16)
    good_out = dev((1, 2, 100, 64), torch.uint8)
    good_sc = dev((1, 2, 2), torch.float32)
    for bad in (dev((1, 2, 99, 64), torch.uint8), dev((1, 2, 100, 64), torch.float16),
                Dev(torch.zeros((1, 2, 100, 64), dtype=torch.uint8), torch.device("cpu"))):
        with pytest.raises(ValueError):
            fa.quantize_fp8(x, 64, out=bad, scales=good_sc)
    for why, bad in _bad_outputs((1, 2, 2), torch.float32):
        with pytest.raises(ValueError):
            fa.quantize_fp8(x, 64, out=good_out, scales=bad)


def test_good_buffers_pass_the_checks():
    """Control: with every buffer right, the calls above get past the checks
    and stop at the stream lookup (no GPU here), so the ValueErrors above come
    from the buffer checks and not from the stand-ins."""
    q = dev(QS)
    B, H, N, d = QS
    calls = [
        lambda: fa.forward(q, q, q, out=dev(QS), lse=dev(QS[:3], torch.float32)),
        lambda: fa.backward(q, q, q, q, dev(QS[:3], torch.float32), q, dq=dev(QS), dk=dev(QS),
                            dv=dev(QS), workspace=dev((2 * B * H * N,), torch.float32)),
        lambda: fa.forward_fp8(dev(QS, torch.uint8), dev(QS, torch.uint8), dev(QS, torch.uint8),
                               (1.0, 1.0, 1.0), out=dev(QS), lse=dev(QS[:3], torch.float32)),
    ]
    for call in calls:
        with pytest.raises(Exception) as e:
            call()
        assert not isinstance(e.value, ValueError), e.value
