"""The C-ABI library on the CPU (no GPU calls): it loads, exports every entry point include/moe.h
declares, and rejects bad arguments with the documented status before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_layer_gemm_amd as moe
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # a non-null address; never dereferenced (every case fails validation first)


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(moe.lib_path()):
        from mixture_experts_layer_gemm_amd.build import build
        build()
    moe.lib()


def _declared(header="moe.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    return set(re.findall(r"^\s*(?:const\s+char\s*\*\s*|size_t\s+|moe_status\s+|int\s+)(moe_\w+)\s*\(", src, flags=re.M))


# The layer's boundary: the five calls of the hot path, the two helpers, the variant of
# moe_layer_forward that allocates nothing, and the MMOE block-level aggregation next to the layer.
LAYER_ABI = {"moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
             "moe_workspace_bytes", "moe_strerror", "moe_layer_forward_noalloc", "moe_attnres_aggregate"}


def _exported():
    """moe_* functions the shared library exports (its dynamic symbol table)."""
    out = subprocess.run(["nm", "-D", "--defined-only", moe.lib_path()], capture_output=True, text=True, check=True)
    return {ln.split()[-1] for ln in out.stdout.splitlines() if ln.split() and ln.split()[-1].startswith("moe_")}


def test_exports_exactly_the_declared_entry_points():
    assert _declared("moe.h") == LAYER_ABI == set(moe.EXPORTS)
    assert _declared("moe_prof.h") == set(moe.PROF_EXPORTS)
    L = ctypes.CDLL(moe.lib_path())
    for n in LAYER_ABI | set(moe.PROF_EXPORTS):
        assert hasattr(L, n), n
    assert _exported() == LAYER_ABI | set(moe.PROF_EXPORTS)


def test_strerror():
    assert moe.moe_strerror(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert moe.moe_strerror(s) != "unknown status"
    assert moe.moe_strerror(-99) == "unknown status"


def test_workspace_sizes_for_workloads():
    for spec in WORKLOADS.values():
        n = moe.moe_workspace_bytes(moe.desc_from_spec(spec))
        assert n >= 256 and n % 256 == 0


def _desc(**kw):
    d = moe.desc_from_spec(WORKLOADS["dit_moe_xl"])
    for k, v in kw.items():
        setattr(d, k, v)
    return d


INVALID = [
    dict(k=0), dict(k=9), dict(S=-1), dict(d=0), dict(E_heavy=-1), dict(dtype=7), dict(act=5), dict(mode=4),
    dict(d_ff=0), dict(reuse_tau=-0.5), dict(reuse_tau=float("nan")), dict(flags=0x1000),
    dict(flags=moe.MOE_F_FORCE_TILED | moe.MOE_F_FORCE_STREAM),
    dict(mode=moe.MOE_DES_VOTE, m_core=0, vote_k=8), dict(mode=moe.MOE_DES_VOTE, m_core=9, vote_k=2),
    dict(mode=moe.MOE_DES_VOTE, m_core=4, vote_k=0),
    dict(mode=moe.MOE_DES_SEQ, vote_k=0), dict(mode=moe.MOE_DES_SEQ, vote_k=9),
    dict(mode=moe.MOE_EXPERT_CHOICE, capacity_factor=0.0),
    dict(mode=moe.MOE_EXPERT_CHOICE, capacity_factor=0.0009),            # C rounds to 0
    dict(E_heavy=0, n_identity=0, n_zero=0, n_const=0),
]

UNSUPPORTED = [
    dict(d=1160),                                   # router needs d % 32 (bf16)
    dict(E_heavy=300),                              # more than 256 routed experts
    dict(k=8, E_heavy=40),                          # fine ...
    dict(k=17, E_heavy=40),                         # ... but k > 16 is not implemented
    dict(mode=moe.MOE_EXPERT_CHOICE, n_zero=1),     # zero-computation experts under expert choice
    dict(d_ff=4600),                                # GEMM tiles need d_ff % 64
    dict(d=1120),                                   # the GEMM's K blocks (up: K = d) need d % 64 in bf16
]


@pytest.mark.parametrize("kw", INVALID)
def test_invalid_descriptors(kw):
    d = _desc(**kw)
    assert moe.moe_workspace_bytes(d) == 0
    st = moe.moe_layer_forward(d, FAKE, moe.MoeWeights(*([FAKE] * 8)), None, None, None, FAKE, None, FAKE, FAKE,
                               1 << 40, stream=0, raise_on_error=False)
    assert st == moe.MOE_EINVAL


@pytest.mark.parametrize("kw", UNSUPPORTED)
def test_unsupported_descriptors(kw):
    d = _desc(**kw)
    if kw == dict(k=8, E_heavy=40):
        assert moe.moe_workspace_bytes(d) > 0
        return
    assert moe.moe_workspace_bytes(d) == 0
    st = moe.moe_layer_forward(d, FAKE, moe.MoeWeights(*([FAKE] * 8)), None, None, None, FAKE, None, FAKE, FAKE,
                               1 << 40, stream=0, raise_on_error=False)
    assert st == moe.MOE_EUNSUPPORTED


@pytest.mark.parametrize("name", ["dit_moe_xl", "ec_dit", "des_vote_b025", "des_seq", "mmoe"])
def test_empty_batch_is_valid_and_launches_nothing(name):
    """S = 0 is a valid description in every mode (expert choice included, whose capacity is then 0).
    Without routing arrays the layer has nothing to write, so it returns at once, with null token
    arrays and no workspace (no HIP call is made: this runs without a GPU)."""
    d = moe.desc_from_spec(WORKLOADS[name].replace(S=0))
    assert moe.moe_workspace_bytes(d) >= 256
    w = moe.MoeWeights(*([FAKE] * 8))
    assert moe.moe_layer_forward(d, None, w, None, None, None, FAKE, None, None, None, 0, stream=0,
                                 raise_on_error=False) == moe.MOE_OK
    assert moe.moe_dispatch(d, None, moe.MoeRouting(), None, stream=0, raise_on_error=False) == moe.MOE_OK
    assert moe.moe_combine(d, None, moe.MoeRouting(), None, None, FAKE, FAKE, None, None, stream=0,
                           raise_on_error=False) == moe.MOE_OK
    assert moe.moe_expert_ffn(d, None, None, moe.MoeRouting(), w, None, None, None, 0, stream=0,
                              raise_on_error=False) == moe.MOE_OK
    # moe_route writes the routing's counts; without routing arrays it is an argument error
    assert moe.moe_route(d, None, moe.MoeRouting(), None, 0, stream=0, raise_on_error=False) == moe.MOE_EINVAL


def test_misaligned_buffers_are_rejected():
    """Buffers read or written 16 bytes at a time must start on a 16-byte boundary: a token array, an
    expert-output array or a weight that does not gives MOE_EINVAL before any launch."""
    d = moe.desc_from_spec(WORKLOADS["dit_moe_xl"])
    bad = FAKE + 8
    good_w = moe.MoeWeights(*([FAKE] * 8))
    bad_w = moe.MoeWeights(*([FAKE] * 8))
    bad_w.w1 = bad
    ws = 1 << 40
    def layer(x=FAKE, y=FAKE, w=good_w, residual=None):
        return moe.moe_layer_forward(d, x, w, None, None, None, FAKE, residual, y, FAKE, ws, stream=0,
                                     raise_on_error=False)
    assert layer(x=bad) == moe.MOE_EINVAL
    assert layer(y=bad) == moe.MOE_EINVAL
    assert layer(residual=bad) == moe.MOE_EINVAL
    assert layer(w=bad_w) == moe.MOE_EINVAL
    r = moe.MoeRouting(*([FAKE] * 15))
    assert moe.moe_dispatch(d, bad, r, FAKE, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert moe.moe_combine(d, FAKE, r, bad, FAKE, None, None, None, FAKE, stream=0,
                           raise_on_error=False) == moe.MOE_EINVAL
    assert moe.moe_expert_ffn(d, FAKE, None, r, good_w, FAKE, bad, FAKE, ws, stream=0,
                              raise_on_error=False) == moe.MOE_EINVAL


def test_null_pointers_and_workspace():
    d = _desc()
    w = moe.MoeWeights(*([FAKE] * 8))
    call = lambda **kw: moe.moe_layer_forward(  # noqa: E731
        d, kw.get("x", FAKE), kw.get("w", w), None, None, None, FAKE, None, kw.get("y", FAKE), kw.get("ws", FAKE),
        kw.get("nb", 1 << 40), stream=0, raise_on_error=False)
    assert call(x=None) == moe.MOE_EINVAL
    assert call(y=None) == moe.MOE_EINVAL
    assert call(w=moe.MoeWeights(None, *([FAKE] * 7))) == moe.MOE_EINVAL          # no router weight
    assert call(w=moe.MoeWeights(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE)) == moe.MOE_EINVAL  # SwiGLU w3
    assert call(ws=None) == moe.MOE_EWORKSPACE
    assert call(nb=1024) == moe.MOE_EWORKSPACE
    assert call(ws=FAKE + 8) == moe.MOE_EWORKSPACE                                 # misaligned
    # the reuse variant needs a cache
    d2 = moe.desc_from_spec(WORKLOADS["dit_moe_xl_reuse"])
    st = moe.moe_layer_forward(d2, FAKE, w, None, None, None, None, None, FAKE, FAKE, 1 << 40, stream=0,
                               raise_on_error=False)
    assert st == moe.MOE_EINVAL
    # probabilities are an input of moe_route only
    d3 = _desc(flags=moe.MOE_F_INPUT_PROBS)
    st = moe.moe_layer_forward(d3, FAKE, w, None, None, None, FAKE, None, FAKE, FAKE, 1 << 40, stream=0,
                               raise_on_error=False)
    assert st == moe.MOE_EINVAL


def test_route_and_combine_argument_checks():
    d = _desc()
    r = moe.MoeRouting()
    assert moe.moe_route(d, FAKE, r, FAKE, 1 << 40, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert moe.moe_route(d, None, r, FAKE, 1 << 40, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    full = moe.MoeRouting(*([FAKE] * 15))
    assert moe.moe_route(d, FAKE, full, FAKE, 16, stream=0, raise_on_error=False) == moe.MOE_EWORKSPACE
    assert moe.moe_dispatch(d, None, full, FAKE, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert moe.moe_combine(d, FAKE, full, None, FAKE, None, None, None, FAKE, stream=0,
                           raise_on_error=False) == moe.MOE_EINVAL       # heavy experts need y_perm
    assert moe.moe_combine(d, FAKE, full, FAKE, None, None, None, None, FAKE, stream=0,
                           raise_on_error=False) == moe.MOE_EINVAL       # shared experts need y_shared
    assert moe.moe_expert_ffn(d, FAKE, None, full, moe.MoeWeights(*([FAKE] * 8)), FAKE, FAKE, FAKE, 16, stream=0,
                              raise_on_error=False) == moe.MOE_EWORKSPACE


def test_binding_raises_with_status():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(_desc(k=0), FAKE, moe.MoeRouting(), FAKE, 1, stream=0)
    assert ei.value.status == moe.MOE_EINVAL


def test_attnres_argument_checks():
    """Invalid arguments are rejected on the host, before anything is launched (no GPU needed)."""
    a, q, o = 0x10000, 0x20000, 0x30000   # never dereferenced: every call below fails validation
    call = moe.moe_attnres_aggregate
    assert call(moe.MOE_BF16, 4, 64, [], q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 64, [a, None], q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 64, [a], None, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 64, [a], q, 1e-6, None, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, -1, 64, [a], q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 0, [a], q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 64, [a], q, -1.0, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 64, [a], q, float("nan"), o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(7, 4, 64, [a], q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 64, [a + 8], q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 64, [a], q + 2, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EINVAL
    assert call(moe.MOE_BF16, 4, 60, [a], q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EUNSUPPORTED
    assert call(moe.MOE_BF16, 4, 8192, [a], q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EUNSUPPORTED
    assert call(moe.MOE_BF16, 4, 64, [a] * 65, q, 1e-6, o, stream=0, raise_on_error=False) == moe.MOE_EUNSUPPORTED
    with pytest.raises(moe.MoeError):
        call(moe.MOE_BF16, 4, 64, [], q, 1e-6, o, stream=0)


def test_noalloc_rejects_before_any_launch():
    """The no-allocation entry point validates on the host: a description whose scratch exceeds the
    static buffer gives MOE_ESCRATCH, an invalid or unsupported one the status moe_layer_forward gives."""
    w = moe.MoeWeights(*([FAKE] * 8))
    big = moe.desc_from_spec(WORKLOADS["dit_moe_xl"])                       # about 397 MiB of scratch
    assert moe.moe_workspace_bytes(big) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert moe.moe_layer_forward_noalloc(big, FAKE, w, None, None, None, None, None, FAKE, stream=0,
                                         raise_on_error=False) == moe.MOE_ESCRATCH
    assert moe.moe_layer_forward_noalloc(_desc(k=0), FAKE, w, None, None, None, None, None, FAKE, stream=0,
                                         raise_on_error=False) == moe.MOE_EINVAL
    assert moe.moe_layer_forward_noalloc(_desc(d=1160), FAKE, w, None, None, None, None, None, FAKE, stream=0,
                                         raise_on_error=False) == moe.MOE_EUNSUPPORTED
