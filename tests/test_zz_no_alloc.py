"""The allocation-free layer call (maple_moe_layer_forward_noalloc), whose
workspace is the library's static device array, against
maple_moe_layer_forward with a caller workspace, on the same seeded inputs.

Both run the same kernels on the same inputs, so routing (top-k indices and
gates, logits, grouping) and outputs must be bitwise equal; a few rows are
also checked against the oracle at the layer tolerance.  The calls come in a
row with shrinking sizes (grouped path, GEMV path, one-token path, fine form),
so that no call may depend on what the previous one left in the shared array.
A call too large for the array is rejected before any launch.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import Layer, assert_close, dims_for, layer_tokens_with_gap, log, x_device  # noqa: E402
from ternary_weight_moe_amd import _native as N  # noqa: E402
from ternary_weight_moe_amd import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu


def call(w, L, x_host, flags, noalloc):
    T, H, E, k = x_host.shape[0], w.hidden, w.n_experts, w.top_k
    d = dims_for(w, flags)
    x = x_device(w, x_host)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    bufs = dict(idx=torch.full((T, k), -1, **i32),
                gate=torch.full((T, k), float("nan"), device="cuda"),
                logits=torch.full((T, E), float("nan"), device="cuda"),
                offsets=torch.full((E + 1,), -1, **i32),
                sorted_token=torch.full((T * k,), -1, **i32),
                slot_pos=torch.full((T, k), -1, **i32))
    if noalloc:
        N.maple_moe_layer_forward_noalloc(d, T, x, L.d_Wr, L.d_bias, L.packed, L.d_alpha, out,
                                          N.make_debug(**bufs))
    else:
        ws = torch.empty(N.maple_moe_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
        N.maple_moe_layer_forward(d, T, x, L.d_Wr, L.d_bias, L.packed, L.d_alpha, out, ws,
                                  N.make_debug(**bufs))
    torch.cuda.synchronize()
    return out.cpu().numpy(), {n: b.cpu().numpy() for n, b in bufs.items()}


def test_noalloc_matches_the_workspace_call():
    w = S.WORKLOADS["decode_layer"]
    L = Layer(w, 0)
    x, _ = layer_tokens_with_gap(w, L, 100, token0=30000)
    d = dims_for(w)
    assert N.maple_moe_workspace_bytes(d, 100) <= N.MAPLE_STATIC_SCRATCH_BYTES
    for T, flags in ((100, 0), (37, 0), (5, 0), (1, 0), (24, N.MAPLE_FINE_LIMBS)):
        log(f"noalloc: T={T} flags={flags:#x}")
        got, gd = call(w, L, x[:T], flags, noalloc=True)
        ref, rd = call(w, L, x[:T], flags, noalloc=False)
        assert np.all(np.isfinite(got)), T
        assert np.array_equal(got, ref), f"T={T}: outputs differ from the workspace call"
        for n in rd:
            assert np.array_equal(gd[n], rd[n], equal_nan=True), f"T={T}: {n} differs"
        rows = np.unique([0, T // 2, T - 1])
        x64 = S.x_as_f32(w, x[:T]).astype(np.float64)[rows]
        assert_close(got[rows], L.oracle_layer(x64, w.top_k, w.inter)["out"], f"noalloc T={T}")


def test_noalloc_rejects_calls_beyond_the_array_and_accepts_empty_ones():
    w = S.WORKLOADS["decode_layer"]
    L = Layer(w, 0)
    d = dims_for(w)
    T = 256
    assert N.maple_moe_workspace_bytes(d, T) > N.MAPLE_STATIC_SCRATCH_BYTES
    x = torch.zeros(T, w.hidden, dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, w.hidden), 3.0, device="cuda")
    with pytest.raises(N.MapleError) as ei:
        N.maple_moe_layer_forward_noalloc(d, T, x, L.d_Wr, None, L.packed, L.d_alpha, out)
    assert ei.value.status == N.MAPLE_ERR_WORKSPACE_TOO_SMALL
    N.maple_moe_layer_forward_noalloc(d, 0, x, L.d_Wr, None, L.packed, L.d_alpha, out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
