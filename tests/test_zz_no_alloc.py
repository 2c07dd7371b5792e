"""h3attn_residual_change_noalloc, the entry point for callers that cannot allocate device memory,
called through the C ABI: two calls in a row (the second on a smaller input) give bit for bit the
results of h3attn_residual_change with a caller workspace; sizes past the device scratch are
refused."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    import video_diffusion_transformer_qk_amd as h3
    return h3.load_library()


def _pair(n, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    prev = torch.randn((n,), generator=g, device=DEV).to(torch.bfloat16)
    cur = (prev.float() + 0.05 * torch.randn((n,), generator=g, device=DEV)).to(torch.bfloat16)
    return cur, prev


def _with_workspace(lib, cur, prev):
    n = cur.numel()
    ws = torch.empty((lib.h3attn_residual_workspace_bytes(n),), dtype=torch.uint8, device=DEV)
    res = torch.empty((2,), dtype=torch.float64, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    assert lib.h3attn_residual_change(cur.data_ptr(), prev.data_ptr(), n, res.data_ptr(), ws.data_ptr(), ws.numel(),
                                      st) == 0
    return res


def test_noalloc_matches_the_workspace_entry_point_on_two_calls(lib):
    st = torch.cuda.current_stream().cuda_stream
    got = []
    # the second call is smaller: it must not see the first call's leftover partial sums
    for n, seed in ((2 * 8192 * 8 * 37 + 5, 1), (8192 * 8 * 3 + 1, 2)):
        cur, prev = _pair(n, seed)
        res = torch.empty((2,), dtype=torch.float64, device=DEV)
        assert lib.h3attn_residual_change_noalloc(cur.data_ptr(), prev.data_ptr(), n, res.data_ptr(), st) == 0, \
            lib.h3attn_last_error().decode()
        want = _with_workspace(lib, cur, prev)
        torch.cuda.synchronize()
        assert res.tolist() == want.tolist(), (n, res.tolist(), want.tolist())
        # and against the plain sums in float64 on the host (the same 1e-6 bar as the workspace path)
        d = (cur.double() - prev.double()).abs().sum().item()
        p = prev.double().abs().sum().item()
        assert abs(res[0].item() - d) <= 1e-6 * d and abs(res[1].item() - p) <= 1e-6 * p
        got.append(res.tolist())
    assert got[0] != got[1]


def test_noalloc_refuses_sizes_past_its_scratch(lib):
    cur, prev = _pair(64, 3)
    res = torch.empty((2,), dtype=torch.float64, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    too_big = (1 << 17) * 8192 * 8 + 1
    assert lib.h3attn_residual_change_noalloc(cur.data_ptr(), prev.data_ptr(), too_big, res.data_ptr(), st) == 1
    assert "allocation-free" in lib.h3attn_last_error().decode()
