"""Host-side checks of the Python binding (CPU only): tensors handed to the C
ABI must be GPU tensors of the flags' dtype, contiguous (except through the
strided entry point) and large enough for M x H; otherwise the binding raises
ValueError before any address reaches the library.

CPU tensors stand in for device memory through a thin proxy that reports a GPU
device; the binding only reads their metadata, never their data, and every
call below is stopped by a check before any address reaches the library.
"""
import pytest
import torch

from all_reduce_residual_rank_amd import arrms


class Dev:
    """A CPU tensor presented as a GPU tensor (metadata only)."""
    is_cuda = True
    device = torch.device("cuda", 0)

    def __init__(self, t):
        self.t = t
        self.dtype = t.dtype
        self.shape = t.shape

    def is_contiguous(self):
        return self.t.is_contiguous()

    def untyped_storage(self):
        return self.t.untyped_storage()

    def storage_offset(self):
        return self.t.storage_offset()

    def element_size(self):
        return self.t.element_size()

    def data_ptr(self):
        return 0  # never reached: every call here fails a check first

    def stride(self, d):
        return self.t.stride(d)

    def dim(self):
        return self.t.dim()

    def numel(self):
        return self.t.numel()


def _args(M=4, H=64, dt=torch.bfloat16, R=2):
    xs = [Dev(torch.zeros(M, H, dtype=dt)) for _ in range(R)]
    return dict(rank_in=xs, residual=Dev(torch.zeros(M, H, dtype=dt)), weight=Dev(torch.zeros(H, dtype=dt)),
                out=Dev(torch.zeros(M, H, dtype=dt)), residual_out=Dev(torch.zeros(M, H, dtype=dt)))


def _fused(a, **kw):
    arrms.arrms_fused(a["rank_in"], a["residual"], a["weight"], a["out"], a["residual_out"],
                      kw.pop("fp8_out", None), kw.pop("fp8_scale", None), eps=1e-6, **kw)


def test_cpu_tensor_is_refused():
    a = _args()
    a["out"] = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        _fused(a, flags=arrms.DTYPE_BF16)


def test_dtype_must_match_flags():
    a = _args()
    with pytest.raises(ValueError, match="float16"):
        _fused(a, flags=arrms.DTYPE_FP16)
    a = _args(dt=torch.float32)
    with pytest.raises(ValueError, match="bfloat16"):
        _fused(a, flags=arrms.DTYPE_BF16)


def test_short_rank_input_is_refused():
    a = _args()
    a["rank_in"][1] = Dev(torch.zeros(3, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"rank_in\[1\] holds"):
        _fused(a, flags=arrms.DTYPE_BF16)
    # a view that starts late in its storage counts only what follows it
    a = _args()
    a["residual_out"] = Dev(torch.zeros(5, 64, dtype=torch.bfloat16)[2:])
    with pytest.raises(ValueError, match="residual_out holds"):
        _fused(a, flags=arrms.DTYPE_BF16, M=4, H=64)


def test_non_contiguous_is_refused_outside_strided():
    a = _args()
    a["residual"] = Dev(torch.zeros(4, 128, dtype=torch.bfloat16)[:, :64])
    with pytest.raises(ValueError, match="contiguous"):
        _fused(a, flags=arrms.DTYPE_BF16)


def test_fp8_buffers_are_sized():
    a = _args()
    with pytest.raises(ValueError, match="fp8_out holds"):
        _fused(a, flags=arrms.DTYPE_BF16 | arrms.FP8, fp8_out=Dev(torch.zeros(4 * 64 - 1, dtype=torch.uint8)),
               fp8_scale=Dev(torch.zeros(4, dtype=torch.float32)))
    with pytest.raises(ValueError, match="fp8_scale holds"):
        _fused(a, flags=arrms.DTYPE_BF16 | arrms.FP8, fp8_out=Dev(torch.zeros(4 * 64, dtype=torch.uint8)),
               fp8_scale=Dev(torch.zeros(3, dtype=torch.float32)))


def test_quant_buffers_are_sized_per_form():
    a = _args(M=2, H=256)
    # MXFP4: [M][H/2] code bytes and [M][H/32] scale bytes
    with pytest.raises(ValueError, match="fp8_scale holds"):
        arrms.arrms_fused_quant(a["rank_in"], a["residual"], a["weight"], None, a["residual_out"],
                                Dev(torch.zeros(2 * 128, dtype=torch.uint8)), Dev(torch.zeros(15, dtype=torch.uint8)),
                                eps=1e-6, flags=arrms.DTYPE_BF16, quant=arrms.QUANT_MXFP4)
    # per-group FP8: [M][H/128] fp32 scales
    with pytest.raises(ValueError, match="fp8_scale holds"):
        arrms.arrms_fused_quant(a["rank_in"], a["residual"], a["weight"], None, a["residual_out"],
                                Dev(torch.zeros(2 * 256, dtype=torch.uint8)), Dev(torch.zeros(3, dtype=torch.float32)),
                                eps=1e-6, flags=arrms.DTYPE_BF16, quant=arrms.QUANT_FP8_GROUP)


def test_strided_checks_the_span():
    a = _args(M=4, H=64)
    # padded rows: stride 128, so 3 * 128 + 64 elements are needed
    big = [Dev(torch.zeros(4, 128, dtype=torch.bfloat16)[:, :64]) for _ in range(2)]
    short = Dev(torch.zeros(3 * 128 + 63, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="residual holds"):
        arrms.arrms_fused_strided(big, short, a["weight"], big[0], big[1], eps=1e-6, flags=arrms.DTYPE_BF16,
                                  M=4, H=64, ld_in=128, ld_residual=128, ld_out=128, ld_residual_out=128)


def test_sum_checks():
    xs = [Dev(torch.zeros(64, dtype=torch.float16)) for _ in range(3)]
    with pytest.raises(ValueError, match="out holds"):
        arrms.arrms_allreduce_sum(xs, Dev(torch.zeros(32, dtype=torch.float16)), flags=arrms.DTYPE_FP16, n=64)
    with pytest.raises(ValueError, match="float16"):
        arrms.arrms_allreduce_sum(xs, Dev(torch.zeros(64, dtype=torch.bfloat16)), flags=arrms.DTYPE_BF16)
