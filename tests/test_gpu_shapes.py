"""GPU parity over every shape class the ABI accepts: hidden 256..4096 and
inter 128..2048 (powers of two), each through every path that serves it.

- One token (T = 1) with automatic dispatch, with and without top-k
  renormalisation: the matrix-core one-token kernels serve hidden 2048/4096
  with inter 256/512; the VALU one-token kernels serve every other shape.
- The VALU GEMV path (forced), T = 5.
- The grouped matrix-core path for inter <= 512 (the grouped kernels' limit),
  T = 40: the fast form, the fine form and the A8 variant.

Every shape has 16 experts and top-4; expert counts that are not multiples
of the kernels' groupings (40, 100, 250) run at hidden 1024, inter 256, and
the small-M chunking at its extremes.  Routing is compared bit-exact and
outputs within the layer tolerances, against the oracle on the same seeded
inputs; tokens obey the router gap rule.  (The architecture table of the
linlog.top article "Maple-Preview" fixes hidden 2048, 256 experts, top-8 and
intermediate 512; the other shapes are the ones the ABI admits besides.)
"""
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import (Layer, check_a8, check_layer, layer_tokens_with_gap,  # noqa: E402
                         log, workload)
from ternary_weight_moe_amd import _native as N  # noqa: E402

pytestmark = pytest.mark.gpu

HIDDEN = (256, 512, 1024, 2048, 4096)
INTER = (128, 256, 512, 1024, 2048)
GROUPED_MAX_INTER = 512


@pytest.mark.parametrize("I", INTER, ids=lambda v: f"i{v}")
@pytest.mark.parametrize("H", HIDDEN, ids=lambda v: f"h{v}")
def test_shape_every_path(H, I):
    w = workload("tiny_layer", name=f"shape_{H}_{I}", hidden=H, inter=I, n_experts=16,
                 top_k=4, n_tokens=40, x_bf16=True, seed=6000 + H + I)
    log(f"shape H={H} I={I}: generating the layer")
    L = Layer(w, 0)
    x1, _ = layer_tokens_with_gap(w, L, 2, token0=100)
    for t in range(2):
        for renorm in (False, True):
            check_layer(w, L, x1[t:t + 1], renorm=renorm,
                        what=f"H={H} I={I} one token #{t} renorm={renorm}")
    x5, _ = layer_tokens_with_gap(w, L, 5, token0=200)
    check_layer(w, L, x5, flags=N.MAPLE_FORCE_GEMV, what=f"H={H} I={I} gemv T=5")
    if I > GROUPED_MAX_INTER:
        return
    x40, _ = layer_tokens_with_gap(w, L, 40, token0=300)
    check_layer(w, L, x40, flags=N.MAPLE_FORCE_GROUPED, what=f"H={H} I={I} grouped fast")
    check_layer(w, L, x40, flags=N.MAPLE_FORCE_GROUPED | N.MAPLE_FINE_LIMBS,
                what=f"H={H} I={I} grouped fine")
    check_a8(w, L, x40, what=f"H={H} I={I} a8")


@pytest.mark.parametrize("a8", [False, True], ids=["fine", "a8"])
def test_small_m_degenerate_routing(a8):
    """The small-M chunking at its extremes, hidden 1024, inter 256, 64
    tokens: E == k (every expert holds all 64 slots: 13 chunks of 5, or 4 of
    16 with one limb) and k = 1 (64 slots over 16 experts)."""
    for E, k in ((8, 8), (16, 1)):
        w = workload("tiny_layer", name=f"small_m_{E}_{k}", hidden=1024, inter=256,
                     n_experts=E, top_k=k, n_tokens=64, x_bf16=True, seed=7100 + E + k)
        L = Layer(w, 0)
        x, _ = layer_tokens_with_gap(w, L, 64, token0=400)
        if a8:
            check_a8(w, L, x, what=f"small-M a8 E={E} k={k}")
        else:
            check_layer(w, L, x, flags=N.MAPLE_FORCE_GROUPED | N.MAPLE_FINE_LIMBS,
                        what=f"small-M fine E={E} k={k}")


@pytest.mark.parametrize("a8", [False, True], ids=["fine", "a8"])
def test_small_m_many_rounds(a8):
    """Hidden 4096, inter 512: one 8-wave small-M gate/up block fits a CU, so
    the grid is the 256 blocks the chip holds, and 64 tokens at top-8 over 128
    experts (about 4 slots each) give some 600 work items with three limbs
    (5-slot chunks) or 500 with one (16-slot chunks): every block groups the
    selections once and takes its items in two or three rounds.
    Routing of all 64 tokens bit-exact, outputs of every fourth token."""
    w = workload("tiny_layer", name=f"small_m_rounds_{'a8' if a8 else 'fine'}", hidden=4096,
                 inter=512, n_experts=128, top_k=8, n_tokens=64, x_bf16=True,
                 seed=7300 + (1 if a8 else 0))
    log(f"small-M rounds a8={a8}: generating the layer")
    L = Layer(w, 0)
    x, _ = layer_tokens_with_gap(w, L, 64, token0=600)
    sample = list(range(0, 64, 4))
    if a8:
        check_a8(w, L, x, sample=sample, what="small-M rounds a8")
    else:
        check_layer(w, L, x, flags=N.MAPLE_FORCE_GROUPED | N.MAPLE_FINE_LIMBS, sample=sample,
                    what="small-M rounds fine")


@pytest.mark.parametrize("E,k", [(40, 6), (100, 8), (250, 8)], ids=lambda v: str(v))
def test_uneven_expert_counts(E, k):
    """Expert counts that are not multiples of the kernels' groupings (16
    experts per small-T router block, 64 per router tile, 64 per routing
    lane set), hidden 1024, inter 256: one token, 23 tokens through the
    small-M fine form, the tiled fast form and A8 (the split-K small-T
    router), and 100 tokens through the large-T router."""
    w = workload("tiny_layer", name=f"uneven_{E}_{k}", hidden=1024, inter=256, n_experts=E,
                 top_k=k, n_tokens=100, x_bf16=True, seed=7300 + E + k)
    L = Layer(w, 0)
    x1, _ = layer_tokens_with_gap(w, L, 1, token0=500)
    check_layer(w, L, x1, what=f"E={E} k={k} one token")
    x23, _ = layer_tokens_with_gap(w, L, 23, token0=600)
    check_layer(w, L, x23, flags=N.MAPLE_FORCE_GROUPED | N.MAPLE_FINE_LIMBS,
                what=f"E={E} k={k} T=23 fine")
    check_layer(w, L, x23, flags=N.MAPLE_FORCE_GROUPED, what=f"E={E} k={k} T=23 fast")
    check_a8(w, L, x23, what=f"E={E} k={k} T=23 a8")
    x100, _ = layer_tokens_with_gap(w, L, 100, token0=700)
    check_layer(w, L, x100, flags=N.MAPLE_FORCE_GROUPED, what=f"E={E} k={k} T=100 fast")
