"""The no-allocation loss entry point against usaf_mse_grad (which takes a
caller workspace): bit-identical loss and dY on two calls in a row, the
second on a smaller input, and refusal of inputs beyond its fixed scratch."""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def capi():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_fine_tuning_amd import capi as c
    return c


def noalloc(capi, shape, Y, tgt, dY, loss, nonfinite):
    fn = capi.lib.usaf_mse_grad_noalloc
    fn.argtypes = [C.c_void_p] * 6 + [C.c_void_p]
    fn.restype = C.c_int32
    return fn(C.byref(shape), Y.data_ptr(), tgt.data_ptr(), dY.data_ptr(), loss.data_ptr(),
              nonfinite.data_ptr(), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("act", [1, 0])
def test_noalloc_loss_equals_workspace_loss(capi, act):
    dt = torch.bfloat16 if act else torch.float32
    gen = torch.Generator(device=DEV)
    gen.manual_seed(90 + act)
    for T, H in ((4096, 4096), (200, 192)):  # the second call is smaller
        say(f"noalloc mse act={act} T={T} H={H}")
        shape = capi.Shape(T, H, 8, 2, 32, act)
        Y = torch.randn(T, H, generator=gen, device=DEV).to(dt)
        tgt = torch.randn(T, H, generator=gen, device=DEV).to(dt)
        dY_ref, dY = torch.empty_like(Y), torch.full_like(Y, 3.0)
        loss_ref = torch.zeros(1, device=DEV)
        loss = torch.full((1,), 5.0, device=DEV)
        nf_ref = torch.zeros(1, dtype=torch.int32, device=DEV)
        nf = torch.zeros(1, dtype=torch.int32, device=DEV)
        ws = torch.empty(capi.workspace_size(capi.WS_FORWARD, shape), dtype=torch.uint8, device=DEV)
        capi.mse_grad(shape, Y, tgt, dY_ref, loss_ref, nf_ref, ws)
        assert noalloc(capi, shape, Y, tgt, dY, loss, nf) == 0
        torch.cuda.synchronize()
        assert torch.equal(loss, loss_ref)
        assert torch.equal(dY.view(torch.int16 if act else torch.int32),
                           dY_ref.view(torch.int16 if act else torch.int32))
        assert int(nf.item()) == 0 and int(nf_ref.item()) == 0
        ref = float(((Y.double() - tgt.double()) ** 2).mean())
        assert abs(float(loss.item()) - ref) <= 1e-5 * ref


def test_noalloc_refuses_inputs_beyond_its_scratch(capi):
    shape = capi.Shape(65536, 8192, 8, 2, 32, 1)  # 2^29 elements > 2^28
    t = torch.empty(1, device=DEV)
    nf = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert noalloc(capi, shape, t, t, t, t, nf) == capi.USAF_ERR_UNSUPPORTED
