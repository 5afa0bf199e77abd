"""spec_lm_head_argmax_noalloc (no workspace argument; the ticket and keys live in a
library-owned device array) against spec_lm_head_argmax with a caller workspace:
the same argmax and maxval bytes on two calls in a row, the second with fewer rows,
and the row limit enforced before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _reference(gdv, hidden, wp, V):
    R = hidden.shape[0]
    am = torch.full((R,), -7, dtype=torch.int32, device=hidden.device)
    mv = torch.full((R,), -7.0, dtype=torch.float32, device=hidden.device)
    gdv.spec_lm_head_argmax(hidden, wp, V, am, mv)
    return am, mv


def _noalloc(gdv, hidden, wp, V):
    R, H = hidden.shape
    am = torch.full((R,), -9, dtype=torch.int32, device=hidden.device)
    mv = torch.full((R,), -9.0, dtype=torch.float32, device=hidden.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = gdv.lib().spec_lm_head_argmax_noalloc(_p(hidden), _p(wp), R, H, V, _p(am), _p(mv), stream)
    assert rc == 0, gdv.lib().spec_last_error()
    return am, mv


@pytest.mark.parametrize("H,V,rows", [(512, 5003, (300, 37)), (4096, 151936, (80, 5))])
def test_noalloc_matches_the_workspace_entry_point(H, V, rows):
    import greedy_draft_verify_amd as gdv
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(H + V)
    w = (torch.randn((V, H), generator=g, device=dev) / H ** 0.5).to(torch.bfloat16)
    wp = gdv.spec_lm_head_pack(w)
    del w
    for R in rows:    # two calls in a row on the same scratch array, the second smaller
        print(f"noalloc lm_head H={H} V={V} R={R}", flush=True)
        hidden = torch.randn((R, H), generator=g, device=dev).to(torch.bfloat16)
        am_n, mv_n = _noalloc(gdv, hidden, wp, V)
        am_r, mv_r = _reference(gdv, hidden, wp, V)
        torch.cuda.synchronize()
        assert torch.equal(am_n, am_r)
        assert torch.equal(mv_n.view(torch.int32), mv_r.view(torch.int32))
        assert int(am_n.min()) >= 0 and int(am_n.max()) < V


def test_noalloc_rejects_rows_beyond_its_scratch():
    import greedy_draft_verify_amd as gdv
    L = gdv.lib()
    p = ctypes.c_void_p(0x1000)
    rc = L.spec_lm_head_argmax_noalloc(p, p, gdv.NOALLOC_MAX_ROWS + 1, 4096, 1000, p, p, None)
    assert rc == -2 and b"exceeds" in L.spec_last_error()
    rc = L.spec_lm_head_argmax_noalloc(p, p, 0, 4096, 1000, p, p, None)
    assert rc == -1
