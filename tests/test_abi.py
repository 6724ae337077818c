"""The C-ABI library loads, exports every declared entry point, and rejects
host-detectable misuse before touching the GPU (CPU only, no kernel launches)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "peagle.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from drafting_draft_expand_amd import _lib
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in peagle.h but not exported"


def test_binding_names_match_abi():
    import drafting_draft_expand_amd as pkg
    for n in ("prepare_draft_batch", "draft_forward", "accept"):
        assert callable(getattr(pkg, n))
        assert f"pe_{n}" in _declared()


def test_status_strings(lib):
    from drafting_draft_expand_amd import _lib
    assert _lib.status_string(0) == "ok"
    assert _lib.status_string(-3) == "workspace too small"


def _desc(**kw):
    from drafting_draft_expand_amd import _lib
    d = dict(hidden=64, vocab=512, n_layers=1, n_q=4, n_kv=2, head_dim=16, inter=128, block_size=16,
             rms_eps=1e-6, rope_theta=1e4, mask_token_id=511, dtype=0)
    d.update(kw)
    return _lib.ModelDesc(**d)


def _fake_weights():
    from drafting_draft_expand_amd import _lib
    p = 0x10000  # 16-byte aligned placeholders: create never dereferences them
    layers = (_lib.LayerWeights * 1)(_lib.LayerWeights(*([p] * 9)))
    w = _lib.Weights(p, p, p, p, p, ctypes.cast(layers, ctypes.POINTER(_lib.LayerWeights)))
    return w, layers


def _create(lib, desc):
    w, keep = _fake_weights()
    h = ctypes.c_void_p()
    st = lib.pe_model_create(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,expect", [
    (dict(block_size=32), -2), (dict(head_dim=48), -2), (dict(hidden=60), -2), (dict(n_q=3), -1),
    (dict(mask_token_id=512), -1), (dict(dtype=7), -2), (dict(rms_eps=0.0), -1), (dict(), 0),
])
def test_model_create_validation(lib, kw, expect):
    st, h = _create(lib, _desc(**kw))
    assert st == expect
    if st == 0:
        lib.pe_model_destroy(h)


def test_calls_reject_bad_arguments_before_launch(lib):
    st, h = _create(lib, _desc())
    assert st == 0
    try:
        P = 0x20000
        # c = 0 and null pointers
        args = [h, 0, 3, 8] + [P] * 7 + [1] + [P] * 10 + [None]
        assert lib.pe_prepare_draft_batch(*args) == -1
        args = [h, 2, 3, 8] + [P] * 6 + [None] + [1] + [P] * 10 + [None]
        assert lib.pe_prepare_draft_batch(*args) == -1
        # misaligned hidden rows
        args = [h, 2, 3, 8] + [P] * 5 + [P + 2] + [P] + [1] + [P] * 10 + [None]
        assert lib.pe_prepare_draft_batch(*args) == -1
        # workspace too small
        need = lib.pe_workspace_bytes(h, 2, 3, 12)
        assert need > 0
        kp = (ctypes.c_void_p * 1)(P)
        fargs = [h, 2, 3, 12] + [P] * 9 + [1, ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(kp, ctypes.c_void_p),
                                           0x40000, need - 1, P, None, None, None]
        assert lib.pe_draft_forward(*fargs) == -3
        # N inconsistent with c*K
        fargs[3] = 5
        assert lib.pe_draft_forward(*fargs) == -1
        assert lib.pe_accept(0, 3, P, P, P, P, None) == -1
        assert lib.pe_accept(2, 3, None, P, P, P, None) == -1
        assert lib.pe_workspace_bytes(h, 0, 3, 12) == 0
        # the device check refuses null pointers and empty batches before any launch
        cargs = [h, 2, 3, 8] + [P] * 6 + [4, P, None]
        bad = list(cargs)
        bad[1] = 0
        assert lib.pe_check_verified_batch(*bad) == -1
        bad = list(cargs)
        bad[11] = None
        assert lib.pe_check_verified_batch(*bad) == -1
    finally:
        lib.pe_model_destroy(h)


def test_expansion_only_model_refuses_forward(lib):
    from drafting_draft_expand_amd import _lib
    d = _desc(n_layers=0)
    w = _lib.Weights(None, None, None, None, 0x10000, None)
    h = ctypes.c_void_p()
    assert lib.pe_model_create(ctypes.byref(d), ctypes.byref(w), ctypes.byref(h)) == 0
    P = 0x20000
    kp = (ctypes.c_void_p * 1)(P)
    fargs = [h, 2, 3, 12] + [P] * 9 + [1, ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(kp, ctypes.c_void_p),
                                       0x40000, 1 << 30, P, None, None, None]
    assert lib.pe_draft_forward(*fargs) == -2
    lib.pe_model_destroy(h)


def test_forward_validation_from_two_threads(lib):
    """The handle is read-only after set-up: two host threads validating
    forward calls on the same model at once see the same statuses (no launch
    happens: every call fails a host check first)."""
    import threading
    st, h = _create(lib, _desc())
    assert st == 0
    P = 0x20000
    kp = (ctypes.c_void_p * 1)(P)
    need = lib.pe_workspace_bytes(h, 2, 3, 12)
    short = [h, 2, 3, 12] + [P] * 9 + [1, ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(kp, ctypes.c_void_p),
                                       0x40000, need - 1, P, None, None, None]
    bad_n = list(short)
    bad_n[3] = 5
    results = [[], []]

    def work(slot):
        for _ in range(2000):
            results[slot].append((lib.pe_draft_forward(*short), lib.pe_draft_forward(*bad_n),
                                  lib.pe_workspace_bytes(h, 2, 3, 12)))

    try:
        ts = [threading.Thread(target=work, args=(i,)) for i in range(2)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        for r in results:
            assert len(r) == 2000 and set(r) == {(-3, -1, need)}
    finally:
        lib.pe_model_destroy(h)


def test_timing_api_without_launches(lib):
    from drafting_draft_expand_amd import _lib
    for k in (_lib.PE_KERNEL_LM_HEAD, _lib.PE_KERNEL_PREPARE, _lib.PE_KERNEL_ATTENTION):
        _lib.timing_enable(k, True)
        assert _lib.timing_read(k) == (0.0, 0, [])
        _lib.timing_enable(k, False)
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.pe_timing_read(7, ctypes.byref(ms), ctypes.byref(n), None, 0) == -1
    assert lib.pe_timing_enable(-1, 1) == -1


def test_noalloc_forward_rejects_batches_beyond_its_scratch(lib):
    """pe_draft_forward_noalloc refuses, before any HIP call, a batch whose
    scratch would exceed the static array (GPT-OSS-20B shape, 64 sequences at
    K = 7: about 200 MiB against 32 MiB)."""
    from drafting_draft_expand_amd import _lib
    d = _desc(hidden=2880, vocab=201088, n_q=64, n_kv=8, head_dim=64, inter=7680, mask_token_id=201087, dtype=1)
    st, h = _create(lib, d)
    assert st == 0
    try:
        P = 0x20000
        kp = (ctypes.c_void_p * 1)(P)
        c, K, N = 64, 7, 896
        assert lib.pe_workspace_bytes(h, c, K, N) > _lib.STATIC_SCRATCH_BYTES
        args = [h, c, K, N] + [P] * 9 + [600, ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(kp, ctypes.c_void_p),
                                         P, None, None, None]
        assert lib.pe_draft_forward_noalloc(*args) == -3
        bad = list(args)
        bad[3] = 100  # fewer rows than c * K
        assert lib.pe_draft_forward_noalloc(*bad) == -1
        assert lib.pe_workspace_bytes(h, 1, 7, 14) <= _lib.STATIC_SCRATCH_BYTES
    finally:
        lib.pe_model_destroy(h)


def _up256(v):
    return (v + 255) // 256 * 256


def _packed_bytes_expected(H, V, n_q, n_kv, d, inter, tile_copies):
    """Bytes of the packed copies as the header lays them out: every projection
    in fragment order (16-row tiles of 32-deep KiB fragments), the LM head
    tile-major (256-row groups), and, with hidden, n_q * d and inter multiples
    of 64, every projection once more tile-major, its rows rounded up to whole
    tiles of its ring (128 x 128 for q/k/v, 256-wide otherwise, a SiLU * up tile
    holding 128 output columns), then to 256-row groups; each region 256-byte
    aligned."""
    qd, kvd = n_q * d, n_kv * d
    mats = [(H, 2 * H), (qd + 2 * kvd, H), (H, qd), (inter, H), (inter, H), (H, inter)]
    total = sum(_up256((nout + 15) // 16 * 16 * k * 2) for nout, k in mats)
    total += _up256((V + 255) // 256 * 256 * H * 2)
    if tile_copies:
        def rows(nout, bn, cols):
            return (nout + cols - 1) // cols * bn
        tiles = [(rows(H, 256, 256), 2 * H), (rows(qd + 2 * kvd, 128, 128), H), (rows(H, 256, 256), qd),
                 (rows(inter, 256, 128), H), (rows(H, 256, 256), inter)]
        total += sum(_up256((r + 255) // 256 * 256 * k * 2) for r, k in tiles)
    return total


@pytest.mark.parametrize("shape,tile_copies", [
    (dict(hidden=2880, vocab=201088, n_q=64, n_kv=8, head_dim=64, inter=7680, mask_token_id=201087), True),
    (dict(hidden=288, vocab=1000, n_q=8, n_kv=2, head_dim=32, inter=320, mask_token_id=999), False),
    (dict(hidden=256, vocab=1000, n_q=8, n_kv=2, head_dim=64, inter=512, mask_token_id=999), True),
])
def test_packed_weights_bytes_follow_the_layouts(lib, shape, tile_copies):
    """pe_packed_weights_bytes against the layouts the header documents: the
    GPT-OSS-shaped drafter (the tile-major projections add about 226 MB), a
    hidden width off the 64 grid (no tile-major projections) and a small
    drafter on it; fp32 models pack nothing."""
    st, h = _create(lib, _desc(dtype=1, **shape))
    assert st == 0
    try:
        got = lib.pe_packed_weights_bytes(h)
        want = _packed_bytes_expected(shape["hidden"], shape["vocab"], shape["n_q"], shape["n_kv"],
                                      shape["head_dim"], shape["inter"], tile_copies)
        assert got == want
        if shape["hidden"] == 2880:
            extra = want - _packed_bytes_expected(2880, 201088, 64, 8, 64, 7680, False)
            assert 225e6 < extra < 227e6
    finally:
        lib.pe_model_destroy(h)
    st, h = _create(lib, _desc(dtype=0, **shape))
    assert st == 0
    try:
        assert lib.pe_packed_weights_bytes(h) == 0
    finally:
        lib.pe_model_destroy(h)
