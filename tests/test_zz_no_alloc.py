"""The entry point that allocates nothing: kd_fa_decode_ragged_noalloc, called through the C
ABI, against kd_fa_decode_ragged (caller's workspace) on the same inputs -- the same output
bits -- on two calls in a row, the second with a smaller input (the scratch array keeps the
first call's partials, which the second must not depend on)."""
import numpy as np
import pytest
import torch

from gpu_util import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

kd = pytest.importorskip("session_decode_step_amd")


def _case(B, H, G, hd, t_kv, cap, seed):
    say(f"noalloc B={B} H={H} G={G} hd={hd} t_kv={t_kv}")
    g = torch.Generator(device="cuda").manual_seed(seed)
    caches = [torch.randn((2, G, cap, hd), generator=g, device="cuda").half() for _ in range(B)]
    q = torch.randn((B, H, hd), generator=g, device="cuda")
    kb = [c[0].data_ptr() for c in caches]
    vb = [c[1].data_ptr() for c in caches]
    scale = hd ** -0.5
    ref = kd.kd_fa_decode_ragged(q, G, kb, vb, t_kv, cap, scale)
    out = torch.full_like(q, float("nan"))
    st = kd.lib().kd_fa_decode_ragged_noalloc(q.data_ptr(), B, H, G, hd, kd._ptrs(kb), kd._ptrs(vb), kd._i32(t_kv),
                                              cap, scale, out.data_ptr(), kd._stream(None))
    assert st == kd.KD_OK, kd.lib().kd_last_error()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
    need = kd.kd_fa_decode_workspace(B, H, hd, t_kv)
    say(f"  equal to the workspace call ({need} bytes of partials)")
    return need


def test_noalloc_equals_workspace_call_twice():
    big = _case(8, 32, 8, 128, [4113] * 4 + [1500, 3000, 777, 4000], 4128, 1)
    small = _case(3, 16, 4, 64, [40, 129, 1], 256, 2)
    assert small < big
