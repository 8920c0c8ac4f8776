"""Host-side bounds check of launch plans (no GPU needed).

Every call checks, before launching, that each byte range its kernels can
touch (derived from the descriptors the way the kernels address memory)
lies inside one workspace buffer of the plan's layout or one caller matrix,
with write permission where it is written. ns_plan_check runs that check on
a plan built for plain addresses, so it can run here:

* the plans of every entry point (batched gram and direct, ragged, tall,
  wide, leading dimensions above n, the Muon step whose final product reads
  the caller's parameter as C, 1 to 64 shards, the benchmark workloads)
  pass;
* each of the planted mistakes (a caller's C read over the padded tile, the
  class of the fault once seen on a 300 x 700 Muon parameter; an unclipped
  output store; a K overrun; a cast past its padded block; a norm pass past
  the input; a shard reduction past its parts; a K-major operand read from
  one K block on; a tile deal that claims one tile more than the launch
  has) is caught.

Caller buffers are laid out back to back, so any overrun runs into a
neighbouring buffer rather than into unmapped space.
"""

import os

import pytest

import newton_schulz_matrix_amd as nsmi
import workloads as W

pytestmark = pytest.mark.skipif(not os.path.exists(nsmi.LIB_PATH),
                                reason="libnsmi.so not built")

ES = {nsmi.NS_DT_F32: 4, nsmi.NS_DT_BF16: 2, nsmi.NS_DT_F16: 2}
PLANTS = range(1, 9)


class Arena:
    """Back-to-back fake device addresses (never dereferenced)."""

    def __init__(self, base=1 << 41):
        self.next = base

    def take(self, rows, ld, cols, dtype):
        addr = self.next
        self.next += ((rows - 1) * ld + cols) * ES[dtype]
        self.next = (self.next + 255) // 256 * 256
        return addr


def matrices(shapes, g_dtype=nsmi.NS_DT_F32, o_dtype=nsmi.NS_DT_F16, pad_g=0, pad_o=0):
    ar, out = Arena(), []
    for m, n in shapes:
        g = ar.take(m, n + pad_g, n, g_dtype)
        o = ar.take(m, n + pad_o, n, o_dtype)
        out.append(nsmi._Matrix(g, g_dtype, m, n, n + pad_g, o, o_dtype, n + pad_o))
    return out


def muon_matrices(shapes, pad=0):
    ar, out = Arena(), []
    for m, n in shapes:
        ld = n + pad
        g = ar.take(m, ld, n, nsmi.NS_DT_F32)
        mo = ar.take(m, ld, n, nsmi.NS_DT_F32)
        p = ar.take(m, ld, n, nsmi.NS_DT_BF16)
        out.append(nsmi._MuonMatrix(g, nsmi.NS_DT_F32, m, n, ld, mo, nsmi.NS_DT_F32, ld,
                                    p, nsmi.NS_DT_BF16, ld, 1.0))
    return out


RAGGED = [(300, 700), (700, 300), (256, 256), (1, 1), (1000, 37), (13, 7)]

CASES = {
    "gram ragged": (nsmi.NS_CHECK_BATCHED, matrices(RAGGED), "gram", 1, (2,)),
    "gram ld>n": (nsmi.NS_CHECK_BATCHED,
                  matrices(RAGGED, nsmi.NS_DT_BF16, nsmi.NS_DT_F32, pad_g=17, pad_o=5),
                  "gram", 1, (1, 3)),
    "direct ragged": (nsmi.NS_CHECK_BATCHED, matrices(RAGGED, nsmi.NS_DT_F16,
                                                      nsmi.NS_DT_BF16), "direct", 1, ()),
    "direct ld>n": (nsmi.NS_CHECK_BATCHED, matrices(RAGGED, pad_g=3, pad_o=40), "direct", 1,
                    ()),
    "sharded wide x7": (nsmi.NS_CHECK_SHARDED, matrices([(300, 1000)]), "gram", 7, (2,)),
    "sharded tall x64": (nsmi.NS_CHECK_SHARDED, matrices([(1000, 300)], pad_g=9), "gram", 64,
                         (1, 3)),
    "muon ragged": (nsmi.NS_CHECK_MUON, muon_matrices([(300, 700), (1000, 300)]), "gram", 1,
                    (2,)),
    "muon ld>n": (nsmi.NS_CHECK_MUON, muon_matrices([(257, 513), (700, 129)], pad=11), "gram",
                  1, (2,)),
}


def check(entry, mats, backend, shards, restarts, plant=0):
    return nsmi.ns_plan_check(entry, mats, backend, shards, nsmi.YOU_COEFFICIENTS, restarts,
                              plant=plant)


@pytest.mark.parametrize("name", sorted(CASES))
def test_plans_pass(name):
    st, msg = check(*CASES[name])
    assert st == nsmi.NS_OK, msg


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("plant", PLANTS)
def test_planted_mistakes_are_caught(name, plant):
    st, msg = check(*CASES[name], plant=plant)
    if st == nsmi.NS_ERR_UNSUPPORTED:
        pytest.skip("no descriptor of this plan takes this mistake")
    assert st == nsmi.NS_ERR_INTERNAL, (st, msg)
    assert "outside" in msg or ":" in msg
    print(f"{name} / plant {plant}: {msg}")


def test_every_plant_applies_somewhere():
    """Each planted mistake finds a place in at least one plan above (so the
    parametrised test cannot pass by skipping everything)."""
    for plant in PLANTS:
        statuses = [check(*c, plant=plant)[0] for c in CASES.values()]
        assert nsmi.NS_ERR_INTERNAL in statuses, plant


def test_unclipped_caller_c_read_is_named():
    """The Muon step's final product reads the caller's parameter as C; read
    over the whole padded tile (256 x 768 for a 300 x 700 matrix) it runs
    past the buffer: the fault class seen once on the GPU."""
    entry, mats, be, sh, rs = CASES["muon ragged"]
    st, msg = check(entry, mats, be, sh, rs, plant=1)
    assert st == nsmi.NS_ERR_INTERNAL
    assert msg.startswith("gemm C") and "read" in msg


@pytest.mark.parametrize("wl", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("backend", ["gram", "direct"])
def test_workload_plans_pass(wl, backend):
    w = W.WORKLOADS[wl]
    dt = nsmi.NS_DT_BF16 if w.dtype == "bf16" else nsmi.NS_DT_F32
    mats = matrices(list(w.shapes), dt, nsmi.NS_DT_F16)
    st, msg = nsmi.ns_plan_check(nsmi.NS_CHECK_BATCHED, mats, backend, 1,
                                 nsmi.COEFFICIENT_SETS[w.coefficients], w.restarts)
    assert st == nsmi.NS_OK, msg


def test_owner_batch_muon_plan_passes():
    w = W.WORKLOADS[4]
    st, msg = check(nsmi.NS_CHECK_MUON, muon_matrices(list(w.shapes)), "gram", 1, (2,))
    assert st == nsmi.NS_OK, msg


def test_many_small_matrices_plan_passes():
    import numpy as np
    rng = np.random.default_rng(77)
    shapes = [(int(rng.integers(1, 300)), int(rng.integers(1, 300))) for _ in range(300)]
    for backend in ("gram", "direct"):
        st, msg = check(nsmi.NS_CHECK_BATCHED, matrices(shapes), backend, 1, (2,))
        assert st == nsmi.NS_OK, msg


def test_small_workspace_and_misaligned_workspace_refused():
    entry, mats, be, sh, rs = CASES["gram ragged"]
    st, _ = nsmi.ns_plan_check(entry, mats, be, sh, nsmi.YOU_COEFFICIENTS, rs, ws_bytes=1024)
    assert st == nsmi.NS_ERR_WORKSPACE
    st, _ = nsmi.ns_plan_check(entry, mats, be, sh, nsmi.YOU_COEFFICIENTS, rs, ws=(1 << 40) + 8)
    assert st == nsmi.NS_ERR_WORKSPACE


def test_kmajor_operand_overrun_is_named():
    """The products by X read it K-major (K x width, by pairs of k rows); read
    one K block further they run past the X buffer, and the check names the
    K-major operand."""
    for name in ("gram ragged", "gram ld>n", "sharded wide x7", "sharded tall x64",
                 "muon ragged"):
        st, msg = check(*CASES[name], plant=7)
        assert st == nsmi.NS_ERR_INTERNAL, (name, st, msg)
        assert "K-major" in msg, (name, msg)
