"""The C-ABI library on a CPU host: it loads, exports every declared symbol,
and rejects bad arguments synchronously before touching the GPU."""
import ctypes
import os
import re

import pytest

import matrix_aware_optimizer_amd as mao

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(muon_[a-z_]+)\s*\(", src)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol():
    lib = mao.load()
    declared = _declared_functions()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(lib, name), name
    # the binding knows every declared symbol's signature, and nothing else
    assert sorted(mao.SIGNATURES) == declared


def test_version_and_status_strings():
    assert mao.muon_version() >= 100
    for code in (0, -1, -2, -3, -4):
        assert mao.muon_status_string(code).startswith("MUON_")
    assert "unknown" in mao.muon_status_string(7)


def _hp(**kw):
    hp, keep = mao.make_hparams(schedule=[(3.4445, -4.775, 2.0315)] * 5, **kw)
    return hp, keep


def _mats(specs):
    arr = (mao.MuonMatrix * len(specs))()
    for i, (w, g, m, r, c) in enumerate(specs):
        arr[i] = mao.MuonMatrix(w, g, m, r, c)
    return arr


FAKE = 1 << 40   # host-side validation never dereferences device pointers


def test_workspace_bytes_is_host_only_and_grows_with_work():
    lib = mao.load()
    hp, keep = _hp(dtype=mao.MUON_BF16)
    one = _mats([(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 2048, 2048)])
    two = _mats([(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 2048, 2048),
                 (FAKE + (3 << 30), FAKE + (4 << 30), FAKE + (5 << 30), 8192, 2048)])
    b1 = lib.muon_workspace_bytes(one, 1, ctypes.byref(hp))
    b2 = lib.muon_workspace_bytes(two, 2, ctypes.byref(hp))
    assert b1 > 0 and b2 > b1
    # the iterate as a bf16 pair (two ping-pong hi copies + lo) + A and B (bf16), at least
    assert b1 >= 2048 * 2048 * (2 + 2 + 2) + 2 * 2048 * 2048 * 2
    # fp32: two fp32 iterates + A and B (fp32)
    hp32, keep32 = _hp(dtype=mao.MUON_F32)
    b32 = lib.muon_workspace_bytes(one, 1, ctypes.byref(hp32))
    assert b32 >= 2048 * 2048 * (4 + 4) + 2 * 2048 * 2048 * 4
    # a skipped matrix (grad NULL) costs nothing
    skip = _mats([(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 2048, 2048),
                  (FAKE + (3 << 30), None, FAKE + (5 << 30), 8192, 2048)])
    assert lib.muon_workspace_bytes(skip, 2, ctypes.byref(hp)) == b1


@pytest.mark.parametrize("case", [
    "null_hp", "bad_dtype", "bad_rule", "steps_high", "steps_neg", "nan_lr", "inf_coeff",
    "neg_eps", "bad_flags", "zero_rows", "null_weight", "overlap", "misaligned", "null_schedule",
    "cols_above_max", "rows_above_max",
])
def test_invalid_arguments_are_rejected_before_any_gpu_work(case):
    lib = mao.load()
    kw = {}
    specs = [(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 64, 96)]
    hp, keep = _hp(dtype=mao.MUON_BF16)
    if case == "bad_dtype":
        hp.dtype = 7
    elif case == "bad_rule":
        hp.scale_rule = 9
    elif case == "steps_high":
        hp.ns_steps = 65
    elif case == "steps_neg":
        hp.ns_steps = -1
    elif case == "nan_lr":
        hp.lr = float("nan")
    elif case == "inf_coeff":
        keep[2] = mao.MuonNsCoeffs(float("inf"), 0.0, 0.0)
    elif case == "neg_eps":
        hp.eps = -1.0
    elif case == "bad_flags":
        hp.flags = 6
    elif case == "zero_rows":
        specs = [(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 0, 96)]
    elif case == "null_weight":
        specs = [(None, FAKE + (1 << 30), FAKE + (2 << 30), 64, 96)]
    elif case == "overlap":
        specs = [(FAKE, FAKE + 64, FAKE + (2 << 30), 64, 96)]
    elif case == "misaligned":
        specs = [(FAKE + 1, FAKE + (1 << 30), FAKE + (2 << 30), 64, 96)]
    elif case == "null_schedule":
        hp.schedule = ctypes.POINTER(mao.MuonNsCoeffs)()
    elif case == "cols_above_max":   # MUON_MAX_DIM = 2^20 is the largest accepted extent
        specs = [(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 1, (1 << 20) + 1)]
    elif case == "rows_above_max":
        specs = [(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), (1 << 20) + 1, 1)]
    arr = _mats(specs)
    hpp = None if case == "null_hp" else ctypes.byref(hp)
    st = lib.muon_step(arr, 1, hpp, ctypes.c_void_p(FAKE + (8 << 30)), 1 << 40, None)
    assert st == mao.MUON_ERR_INVALID_ARG, (case, st, mao.muon_last_error_message())
    assert mao.muon_last_error_message() != ""
    assert lib.muon_workspace_bytes(arr, 1, hpp) == 0


def test_maximum_dimension_is_accepted():
    """An extent of exactly MUON_MAX_DIM (2^20), wide or tall, passes validation and
    gets a workspace size (host-only call)."""
    lib = mao.load()
    hp, keep = _hp(dtype=mao.MUON_BF16)
    for rows, cols in ((1, 1 << 20), (1 << 20, 1), (40, 1 << 20)):
        arr = _mats([(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), rows, cols)])
        assert lib.muon_workspace_bytes(arr, 1, ctypes.byref(hp)) > 0, (rows, cols, mao.muon_last_error_message())


def test_workspace_errors():
    lib = mao.load()
    hp, keep = _hp(dtype=mao.MUON_BF16)
    arr = _mats([(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 64, 96)])
    need = lib.muon_workspace_bytes(arr, 1, ctypes.byref(hp))
    ws = FAKE + (8 << 30)
    assert lib.muon_step(arr, 1, ctypes.byref(hp), None, need, None) == mao.MUON_ERR_WORKSPACE
    assert lib.muon_step(arr, 1, ctypes.byref(hp), ctypes.c_void_p(ws), need - 1, None) == mao.MUON_ERR_WORKSPACE
    assert lib.muon_step(arr, 1, ctypes.byref(hp), ctypes.c_void_p(ws + 16), need, None) == mao.MUON_ERR_WORKSPACE
    # a workspace overlapping a matrix is an argument error
    st = lib.muon_step(arr, 1, ctypes.byref(hp), ctypes.c_void_p(FAKE), need, None)
    assert st == mao.MUON_ERR_INVALID_ARG


def test_empty_list_and_all_skipped_are_noops():
    lib = mao.load()
    hp, keep = _hp(dtype=mao.MUON_F32)
    assert lib.muon_step(None, 0, ctypes.byref(hp), None, 0, None) == mao.MUON_OK
    arr = _mats([(FAKE, None, FAKE + (2 << 30), 64, 96)])
    assert lib.muon_step(arr, 1, ctypes.byref(hp), None, 0, None) == mao.MUON_OK


def test_ns_entry_validation():
    lib = mao.load()
    hp, keep = _hp(dtype=mao.MUON_BF16)
    arr = (mao.MuonNsMatrix * 1)()
    arr[0] = mao.MuonNsMatrix(FAKE, FAKE + 8, 16, 16)          # in and out overlap
    assert lib.muon_ns(arr, 1, ctypes.byref(hp), ctypes.c_void_p(FAKE + (8 << 30)), 1 << 40, None) \
        == mao.MUON_ERR_INVALID_ARG
    arr[0] = mao.MuonNsMatrix(FAKE, FAKE + (1 << 30) + 2, 16, 16)  # fp32 out misaligned
    assert lib.muon_ns(arr, 1, ctypes.byref(hp), ctypes.c_void_p(FAKE + (8 << 30)), 1 << 40, None) \
        == mao.MUON_ERR_INVALID_ARG
    arr[0] = mao.MuonNsMatrix(FAKE, FAKE + (1 << 30), 16, 16)
    assert lib.muon_ns_workspace_bytes(arr, 1, ctypes.byref(hp)) > 0


def test_binding_rejects_non_2d_and_non_contiguous():
    torch = pytest.importorskip("torch")
    w = torch.zeros(4, 4, 4)
    with pytest.raises(ValueError):
        mao.muon_workspace_bytes([w], [w], [w], schedule=[(1.0, 0.0, 0.0)])
    w2 = torch.zeros(8, 6).t()
    with pytest.raises(ValueError):
        mao.muon_workspace_bytes([w2], [w2], [w2], schedule=[(1.0, 0.0, 0.0)])


# ----------------------------------------------------------------------------
# AdamW entry points
# ----------------------------------------------------------------------------

def _adamw(specs):
    arr = (mao.MuonAdamwTensor * max(1, len(specs)))()
    for i, (p, g, m, v, n) in enumerate(specs):
        arr[i] = mao.MuonAdamwTensor(p, g, m, v, n)
    return arr


def _adamw_hp(**kw):
    base = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=1, dtype=mao.MUON_BF16)
    base.update(kw)
    return mao.MuonAdamwHparams(base["lr"], base["beta1"], base["beta2"], base["eps"], base["weight_decay"],
                                base["step"], base["dtype"])


GOOD = (FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), 1000)


@pytest.mark.parametrize("case", ["null_hp", "bad_dtype", "beta1_one", "beta2_neg", "nan_lr", "inf_wd", "neg_eps",
                                  "step_zero", "numel_zero", "null_param", "misaligned_moment", "overlap",
                                  "moment_overlaps_param"])
def test_adamw_invalid_arguments_are_rejected(case):
    lib = mao.load()
    spec = list(GOOD)
    hp = _adamw_hp()
    if case == "bad_dtype":
        hp.dtype = 5
    elif case == "beta1_one":
        hp.beta1 = 1.0
    elif case == "beta2_neg":
        hp.beta2 = -0.1
    elif case == "nan_lr":
        hp.lr = float("nan")
    elif case == "inf_wd":
        hp.weight_decay = float("inf")
    elif case == "neg_eps":
        hp.eps = -1e-8
    elif case == "step_zero":
        hp.step = 0
    elif case == "numel_zero":
        spec[4] = 0
    elif case == "null_param":
        spec[0] = None
    elif case == "misaligned_moment":
        spec[2] = FAKE + (2 << 30) + 2
    elif case == "overlap":
        spec[3] = FAKE + (2 << 30) + 8    # the two moments overlap
    elif case == "moment_overlaps_param":
        spec[2] = FAKE + 16
    arr = _adamw([tuple(spec)])
    hpp = None if case == "null_hp" else ctypes.byref(hp)
    st = lib.muon_adamw_step(arr, 1, hpp, ctypes.c_void_p(FAKE + (8 << 30)), 1 << 40, None)
    assert st == mao.MUON_ERR_INVALID_ARG, (case, st, mao.muon_last_error_message())
    assert lib.muon_adamw_workspace_bytes(arr, 1, hpp) == 0


def test_adamw_workspace_errors_and_noops():
    lib = mao.load()
    hp = _adamw_hp()
    arr = _adamw([GOOD, (FAKE + (4 << 30), FAKE + (5 << 30), FAKE + (6 << 30), FAKE + (7 << 30), 77)])
    need = lib.muon_adamw_workspace_bytes(arr, 2, ctypes.byref(hp))
    assert need >= 256
    ws = FAKE + (8 << 30)
    assert lib.muon_adamw_step(arr, 2, ctypes.byref(hp), None, need, None) == mao.MUON_ERR_WORKSPACE
    assert lib.muon_adamw_step(arr, 2, ctypes.byref(hp), ctypes.c_void_p(ws), need - 1, None) == mao.MUON_ERR_WORKSPACE
    assert lib.muon_adamw_step(arr, 2, ctypes.byref(hp), ctypes.c_void_p(ws + 8), need, None) == mao.MUON_ERR_WORKSPACE
    assert lib.muon_adamw_step(arr, 2, ctypes.byref(hp), ctypes.c_void_p(FAKE), need, None) == mao.MUON_ERR_INVALID_ARG
    # empty list and all-skipped lists do nothing
    assert lib.muon_adamw_step(None, 0, ctypes.byref(hp), None, 0, None) == mao.MUON_OK
    skip = _adamw([(FAKE, None, FAKE + (2 << 30), FAKE + (3 << 30), 1000)])
    assert lib.muon_adamw_step(skip, 1, ctypes.byref(hp), None, 0, None) == mao.MUON_OK


def _cayley_mats(specs):
    arr = (mao.MuonCayleyMatrix * len(specs))()
    for i, (w, g, m, r, c) in enumerate(specs):
        arr[i] = mao.MuonCayleyMatrix(w, g, m, r, c)
    return arr


@pytest.mark.parametrize("case", [
    "null_hp", "beta_high", "beta_neg", "beta_nan", "nan_lr", "zero_cols", "null_weight", "null_momentum",
    "overlap", "misaligned",
])
def test_cayley_invalid_arguments_are_rejected(case):
    lib = mao.load()
    specs = [(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 512, 64)]
    hp = mao.MuonCayleyHparams(1e-3, 0.9)
    if case == "beta_high":
        hp.beta = 1.0
    elif case == "beta_neg":
        hp.beta = -0.1
    elif case == "beta_nan":
        hp.beta = float("nan")
    elif case == "nan_lr":
        hp.lr = float("inf")
    elif case == "zero_cols":
        specs = [(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 512, 0)]
    elif case == "null_weight":
        specs = [(None, FAKE + (1 << 30), FAKE + (2 << 30), 512, 64)]
    elif case == "null_momentum":
        specs = [(FAKE, FAKE + (1 << 30), None, 512, 64)]
    elif case == "overlap":
        # momentum starts inside the weight
        specs = [(FAKE, FAKE + (1 << 30), FAKE + 4096, 512, 64)]
    elif case == "misaligned":
        specs = [(FAKE, FAKE + (1 << 30) + 2, FAKE + (2 << 30), 512, 64)]
    arr = _cayley_mats(specs)
    hpp = None if case == "null_hp" else ctypes.byref(hp)
    st = lib.muon_cayley_step(arr, 1, hpp, ctypes.c_void_p(FAKE + (8 << 30)), 1 << 40, None)
    assert st == mao.MUON_ERR_INVALID_ARG, (case, st, mao.muon_last_error_message())
    assert mao.muon_last_error_message() != ""
    assert lib.muon_cayley_workspace_bytes(arr, 1, hpp) == 0


def test_cayley_size_limit_and_workspace_errors():
    lib = mao.load()
    hp = mao.MuonCayleyHparams(1e-3, 0.9)
    # min(rows, cols) above the limit is unsupported, in either orientation
    for r, c in ((4096, 257), (257, 4096)):
        arr = _cayley_mats([(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), r, c)])
        st = lib.muon_cayley_step(arr, 1, ctypes.byref(hp), ctypes.c_void_p(FAKE + (8 << 30)), 1 << 40, None)
        assert st == mao.MUON_ERR_UNSUPPORTED, (r, c, st)
        assert lib.muon_cayley_workspace_bytes(arr, 1, ctypes.byref(hp)) == 0
    # the limit itself is accepted by the host checks
    arr = _cayley_mats([(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 4096, 256)])
    need = lib.muon_cayley_workspace_bytes(arr, 1, ctypes.byref(hp))
    assert need > 0
    ws = FAKE + (8 << 30)
    assert lib.muon_cayley_step(arr, 1, ctypes.byref(hp), None, need, None) == mao.MUON_ERR_WORKSPACE
    assert lib.muon_cayley_step(arr, 1, ctypes.byref(hp), ctypes.c_void_p(ws), need - 1, None) == mao.MUON_ERR_WORKSPACE
    assert lib.muon_cayley_step(arr, 1, ctypes.byref(hp), ctypes.c_void_p(ws + 16), need, None) == mao.MUON_ERR_WORKSPACE
    # a workspace overlapping a matrix is an argument error
    st = lib.muon_cayley_step(arr, 1, ctypes.byref(hp), ctypes.c_void_p(FAKE + (1 << 30)), need, None)
    assert st == mao.MUON_ERR_INVALID_ARG
    # empty list and all-skipped lists do nothing and succeed without a workspace
    assert lib.muon_cayley_step(None, 0, ctypes.byref(hp), None, 0, None) == mao.MUON_OK
    skip = _cayley_mats([(FAKE, None, FAKE + (2 << 30), 512, 64)])
    assert lib.muon_cayley_step(skip, 1, ctypes.byref(hp), None, 0, None) == mao.MUON_OK


def test_noalloc_entry_validation_is_host_side():
    lib = mao.load()
    hp, keep = _hp(dtype=mao.MUON_BF16)
    # empty and all-skipped lists succeed without touching the GPU
    assert lib.muon_step_noalloc(None, 0, ctypes.byref(hp), None) == mao.MUON_OK
    skip = _mats([(FAKE, None, FAKE + (2 << 30), 2048, 2048)])
    assert lib.muon_step_noalloc(skip, 1, ctypes.byref(hp), None) == mao.MUON_OK
    # the same argument checks as muon_step
    assert lib.muon_step_noalloc(_mats([(None, FAKE + (1 << 30), FAKE + (2 << 30), 64, 96)]), 1,
                                 ctypes.byref(hp), None) == mao.MUON_ERR_INVALID_ARG
    assert lib.muon_step_noalloc(_mats([(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 64, 96)]), 1,
                                 None, None) == mao.MUON_ERR_INVALID_ARG
    # a list needing more workspace than the library's array is refused before anything runs
    big = _mats([(FAKE + (k << 32), FAKE + (k << 32) + (1 << 30), FAKE + (k << 32) + (2 << 30), 2048, 8192)
                 for k in range(4)])
    assert lib.muon_workspace_bytes(big, 4, ctypes.byref(hp)) > mao.NOALLOC_SCRATCH_BYTES
    assert lib.muon_step_noalloc(big, 4, ctypes.byref(hp), None) == mao.MUON_ERR_WORKSPACE
    assert "128" in mao.muon_last_error_message() or str(mao.NOALLOC_SCRATCH_BYTES) in mao.muon_last_error_message()
    # the header's limit and the binding's agree
    src = open(HEADER).read()
    assert "#define MUON_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in src
    assert mao.NOALLOC_SCRATCH_BYTES == 128 << 20
