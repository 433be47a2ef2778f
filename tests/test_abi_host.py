"""Host-only checks of libsignmuon.so: it loads, exports every function that
include/signmuon.h declares, and rejects bad arguments before touching the
GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from distributed_bit_matrix_amd import binding as B
from distributed_bit_matrix_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libsignmuon.so not built")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "signmuon.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(signmuon_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 19
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTS)


def test_version_and_strerror():
    L = B.lib()
    assert L.signmuon_abi_version() == 2
    for code in [0, -1, -2, -3, -4, -5, -6]:
        assert len(B.strerror(code)) >= 2
    assert B.strerror(-99) == "unknown status"


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first


def test_apply_validation():
    L = B.lib()
    assert L.signmuon_apply(FAKE, 0, None, None, 0.1, 10, None) == B.SM_EINVAL
    assert L.signmuon_apply(FAKE, 0, FAKE, FAKE, 0.1, 10, None) == B.SM_EINVAL
    assert L.signmuon_apply(FAKE, 2, FAKE, None, 0.1, 10, None) == B.SM_EINVAL
    assert L.signmuon_apply(FAKE, 0, FAKE, None, 0.1, -1, None) == B.SM_EINVAL
    assert L.signmuon_apply(FAKE, 0, FAKE, None, float("nan"), 4, None) == B.SM_EINVAL
    assert L.signmuon_apply(FAKE, 0, FAKE, None, 0.1, 0, None) == B.SM_OK  # no-op


def test_vote_validation():
    L = B.lib()
    assert L.signmuon_majority_vote(FAKE, 1, 0, 32, 0, FAKE, None, None) == B.SM_ERANGE
    assert L.signmuon_majority_vote(FAKE, 1, 32768, 32, 0, FAKE, None, None) == B.SM_ERANGE
    assert L.signmuon_majority_vote(FAKE, 1, 3, 32, 2, FAKE, None, None) == B.SM_EINVAL
    assert L.signmuon_majority_vote(FAKE, 1, 3, 64, 0, FAKE, None, None) == B.SM_EINVAL
    assert L.signmuon_majority_vote(None, 1, 3, 32, 0, FAKE, None, None) == B.SM_EINVAL
    assert L.signmuon_majority_vote(FAKE, 1, 3, 0, 0, FAKE, None, None) == B.SM_OK


def test_momentum_and_pack_validation():
    L = B.lib()
    assert L.signmuon_momentum(FAKE, FAKE, 0, FAKE, 8, 1.0, 0.0, None) == B.SM_EINVAL
    assert L.signmuon_momentum(FAKE, FAKE, 0, FAKE, 8, 0.9, -1.0, None) == B.SM_EINVAL
    assert L.signmuon_momentum(FAKE, FAKE, 5, FAKE, 8, 0.9, 0.0, None) == B.SM_EINVAL
    assert L.signmuon_momentum(None, FAKE, 0, FAKE, 8, 0.9, 0.0, None) == B.SM_EINVAL
    assert L.signmuon_sign_pack(FAKE, FAKE, -3, None) == B.SM_EINVAL
    assert L.signmuon_sign_pack(None, FAKE, 3, None) == B.SM_EINVAL
    assert L.signmuon_sign_pack(FAKE, FAKE, 0, None) == B.SM_OK


def _hp(**kw):
    return B.HParams(**kw)


def test_polar_workspace_gram_space(monkeypatch):
    # the Gram-space form (bfloat16 cubic) adds five Rp x Rp bfloat16 buffers
    hp = _hp(K=5, scale="fro")
    gram = B.polar_ns_workspace(256, 512, hp)
    monkeypatch.setenv("SIGNMUON_NS_FORM", "iterate")
    it = B.polar_ns_workspace(256, 512, hp)
    assert gram - it == 5 * 256 * 256 * 2
    # not used for split-bfloat16, float32, the quintic or the spectral scale
    for kw in [dict(precision="bf16x3"), dict(precision="f32"),
               dict(coeffs=(3.4445, -4.775, 2.0315)), dict(scale="spectral", P=3)]:
        a = B.polar_ns_workspace(256, 512, _hp(K=5, **kw))
        monkeypatch.delenv("SIGNMUON_NS_FORM")
        assert B.polar_ns_workspace(256, 512, _hp(K=5, **kw)) == a
        monkeypatch.setenv("SIGNMUON_NS_FORM", "iterate")


def test_polar_workspace_and_validation(monkeypatch):
    # sizes of the iterate form (the Gram-space form is checked above)
    monkeypatch.setenv("SIGNMUON_NS_FORM", "iterate")
    L = B.lib()
    hp = _hp(K=5, scale="fro")
    w = B.polar_ns_workspace(256, 512, hp)
    assert w > 0 and w % 256 == 0
    assert B.polar_ns_workspace(512, 256, hp) == w            # transposed shape
    assert B.polar_ns_workspace(256, 512, _hp(K=5, precision="bf16x3")) > w
    assert B.polar_ns_workspace(256, 512, _hp(K=5, scale="spectral", P=3)) > w
    assert B.polar_ns_workspace(256, 512, _hp(K=5, coeffs=(3.4445, -4.775, 2.0315))) > w
    assert B.polar_ns_workspace(256, 512, _hp(K=0)) < w
    # invalid hyper-parameters or shapes give 0
    assert B.polar_ns_workspace(0, 512, hp) == 0
    assert B.polar_ns_workspace(256, 512, _hp(eps=0.0)) == 0
    assert B.polar_ns_workspace(256, 512, _hp(scale="spectral", P=0)) == 0
    assert B.polar_ns_workspace(256, 512, _hp(K=65)) == 0
    # size limits: dimensions up to 2^20; padded rows * cols below 2^31
    # (2^30 for float32 Newton-Schulz operands, addressed with 32-bit byte offsets)
    assert B.polar_ns_workspace(1, (1 << 20) + 1, hp) == 0
    assert B.polar_ns_workspace(32768, 32768, hp) > 0
    assert B.polar_ns_workspace(32768, 32768, _hp(K=5, precision="f32")) == 0
    assert B.polar_ns_workspace(32768, 32640, _hp(K=5, precision="f32")) > 0
    assert B.polar_ns_workspace(65536, 32768, hp) == 0
    # long k with one Gram tile: the Gram is split 8 ways along k, with a
    # float32 128x128 partial tile per split in the workspace
    ws_long = B.polar_ns_workspace(128, 4096, hp)
    assert ws_long >= 2 * 2 * 128 * 4096 + 8 * 128 * 128 * 4
    assert ws_long < 2 * 2 * 128 * 4096 + 9 * 128 * 128 * 4 + 64 * 1024
    c = hp.to_c()
    U = ctypes.c_void_p(0x20000)
    assert L.signmuon_polar_ns(FAKE, U, 256, 512, ctypes.byref(c), None, FAKE, 16,
                               None) == B.SM_EWORKSPACE
    assert L.signmuon_polar_ns(FAKE, U, 256, 512, ctypes.byref(c), None,
                               ctypes.c_void_p(0x10010), w, None) == B.SM_EWORKSPACE
    assert L.signmuon_polar_ns(FAKE, FAKE, 256, 512, ctypes.byref(c), None, FAKE, w,
                               None) == B.SM_EINVAL              # X aliases U
    c.ns_precision = 7
    assert L.signmuon_polar_ns(FAKE, ctypes.c_void_p(0x20000), 256, 512, ctypes.byref(c),
                               None, FAKE, w, None) == B.SM_EINVAL


def _step(L, mats, hp, M=3, local=0, stride=None, post=0, ws_bytes=None, G=FAKE):
    arr = B.mats_array(mats)
    if stride is None:
        stride = sum((r * c + 31) // 32 for r, c, _, _ in mats)
    if ws_bytes is None:
        ws_bytes = B.step_workspace(mats, hp, post)
    return L.signmuon_step(arr, len(mats), ctypes.byref(hp.to_c()), G, FAKE, 1, FAKE,
                           FAKE, stride, M, local, post, None, FAKE, ws_bytes, None, None)


def test_worker_pipeline_validation():
    # the per-worker half of the step validates like the step itself
    L = B.lib()
    hp = _hp()
    mats, d, words = B.default_layout([(64, 96), (96, 64)])
    arr = B.mats_array(mats)
    ws = B.step_workspace(mats, hp, False)

    def call(M=3, worker=0, post=0, G=FAKE, stride=words, ws_bytes=ws):
        return L.signmuon_worker_pipeline(arr, len(mats), ctypes.byref(hp.to_c()), G, FAKE, 1,
                                          FAKE, FAKE, stride, M, worker, post, None, FAKE,
                                          ws_bytes, None, None)
    assert call(M=0) == B.SM_ERANGE
    assert call(worker=3) == B.SM_EINVAL
    assert call(worker=-1) == B.SM_EINVAL
    assert call(post=4) == B.SM_EINVAL
    assert call(post=-1) == B.SM_EINVAL
    assert call(G=None) == B.SM_EINVAL
    assert call(stride=words - 1) == B.SM_EINVAL
    assert call(ws_bytes=1024) == B.SM_EWORKSPACE


def test_step_validation():
    L = B.lib()
    hp = _hp()
    mats, d, words = B.default_layout([(64, 96), (96, 64)])
    assert _step(L, mats, hp, M=0) == B.SM_ERANGE
    assert _step(L, mats, hp, M=40000) == B.SM_ERANGE
    assert _step(L, mats, hp, M=3, local=3) == B.SM_EINVAL
    assert _step(L, mats, hp, post=4) == B.SM_EINVAL
    assert _step(L, mats, hp, post=-1) == B.SM_EINVAL
    assert _step(L, mats, hp, G=None) == B.SM_EINVAL
    assert _step(L, mats, hp, stride=words - 1) == B.SM_EINVAL
    overlap = [mats[0], (96, 64, 64 * 96 - 1, mats[1][3])]
    assert _step(L, overlap, hp) == B.SM_EINVAL
    overlap_w = [mats[0], (96, 64, mats[1][2], mats[1][3] - 1)]
    assert _step(L, overlap_w, hp) == B.SM_EINVAL
    assert _step(L, mats, hp, ws_bytes=1024) == B.SM_EWORKSPACE
    assert _step(L, mats, _hp(beta=1.0)) == B.SM_EINVAL
    assert _step(L, mats, _hp(tie_value=2)) == B.SM_EINVAL
    assert _step(L, [(0, 5, 0, 0)], hp) == B.SM_EINVAL


def test_step_workspace_post_vote_modes():
    # 0: Algorithm 2; 1: polar after the vote; 2: both (the pre-sign pass
    # of 0, then the post-vote pass of 1 in the same buffers)
    hp = _hp()
    mats, _, _ = B.default_layout(WL.get("nanogpt").mats)
    assert B.step_workspace(mats, hp, 2) == B.step_workspace(mats, hp, 0) > 0
    assert B.step_workspace(mats, hp, 1) > 0
    assert B.step_workspace(mats, hp, 4) == 0
    assert B.step_workspace(mats, hp, -1) == 0
    # widths that are not multiples of 32 pack their signs in the last
    # epilogue as well (no float32 U in the workspace): the pre-sign modes
    # need no more than the post-vote one
    m1, _, _ = B.default_layout([(5, 37)])
    assert B.step_workspace(m1, hp, 2) == B.step_workspace(m1, hp, 0) == \
        B.step_workspace(m1, hp, 1) > 0


def test_step_workspace_sizes(monkeypatch):
    w = WL.get("nanogpt")
    mats, d, words = B.default_layout(w.mats)
    hp = _hp()
    gram = B.step_workspace(mats, hp, False)
    monkeypatch.setenv("SIGNMUON_NS_FORM", "iterate")
    ws = B.step_workspace(mats, hp, False)
    # Gram-space buffers: five bfloat16 Rp x Rp per matrix
    assert gram - ws == 5 * 2 * sum(min(a, b) ** 2 for a, b in w.mats)
    # two bfloat16 iterates of every matrix (ping-pong), plus the Gram-sized
    # factor
    x = 2 * 2 * d
    r = 2 * sum(min(a, b) ** 2 for a, b in w.mats)
    assert x + r <= ws <= x + r + 4 * 1024 * 1024
    assert B.step_workspace(mats, _hp(K=0), False) < ws
    assert B.step_workspace(mats[:4], hp, False) < ws
    # ragged shapes are padded to multiples of 128
    m1, _, _ = B.default_layout([(10, 2048)])
    assert B.step_workspace(m1, hp, False) >= 2 * 2 * 128 * 2048


def test_ternary_validation():
    # argument errors return before any launch
    L = B.lib()
    F2 = ctypes.c_void_p(0x20000)
    assert L.signmuon_sign_ternary(FAKE, F2, -1, None) == B.SM_EINVAL
    assert L.signmuon_sign_ternary(None, F2, 5, None) == B.SM_EINVAL
    assert L.signmuon_sign_ternary(FAKE, None, 5, None) == B.SM_EINVAL
    assert L.signmuon_sign_ternary(None, None, 0, None) == B.SM_OK
    assert L.signmuon_sign_ternary(FAKE, F2, (1 << 36) + 1, None) == B.SM_EINVAL
    v = L.signmuon_majority_vote_ternary
    assert v(FAKE, 10, 0, 10, 0, F2, None, None) == B.SM_ERANGE
    assert v(FAKE, 10, 32768, 10, 0, F2, None, None) == B.SM_ERANGE
    assert v(FAKE, 10, 3, 10, 2, F2, None, None) == B.SM_EINVAL
    assert v(FAKE, 10, 3, -1, 0, F2, None, None) == B.SM_EINVAL
    assert v(FAKE, 9, 3, 10, 0, F2, None, None) == B.SM_EINVAL      # stride < n
    assert v(None, 10, 3, 10, 0, F2, None, None) == B.SM_EINVAL
    assert v(FAKE, 10, 3, 10, 0, None, None, None) == B.SM_EINVAL
    assert v(None, 0, 3, 0, 0, None, None, None) == B.SM_OK



def test_executor_arguments():
    # a NULL destination is an argument error; destroying NULL is a no-op
    L = B.lib()
    assert L.signmuon_executor_create(None) == B.SM_EINVAL
    assert L.signmuon_executor_destroy(None) == B.SM_OK
    assert L.signmuon_reset_status(None, None) == B.SM_EWORKSPACE
    assert L.signmuon_reset_status(ctypes.c_void_p(0x10010), None) == B.SM_EWORKSPACE


def test_polar_ns_static_limits():
    # argument errors and sizes past the scratch array return before any
    # device work
    L = B.lib()
    hp = _hp(K=5, scale="fro")
    c = hp.to_c()
    U = ctypes.c_void_p(0x20000)
    f = L.signmuon_polar_ns_static
    assert f(FAKE, U, 0, 512, ctypes.byref(c), None, None) == B.SM_EINVAL
    assert f(FAKE, FAKE, 256, 512, ctypes.byref(c), None, None) == B.SM_EINVAL
    assert B.polar_ns_workspace(4096, 4096, hp) > B.STATIC_SCRATCH_BYTES
    assert f(FAKE, U, 4096, 4096, ctypes.byref(c), None, None) == B.SM_ERANGE
    assert B.polar_ns_workspace(1024, 4096, hp) <= B.STATIC_SCRATCH_BYTES
    assert B.polar_ns_workspace(3072, 768, hp) <= B.STATIC_SCRATCH_BYTES


def test_step_ternary_validation():
    # int8 sign buffers: the stride counts bytes and must cover every
    # matrix's elem_off + rows * cols; word_off is not used; an unknown
    # encoding is an argument error
    L = B.lib()
    hp = _hp(encoding="ternary")
    mats, d, words = B.default_layout([(64, 96), (96, 64)])
    assert _step(L, mats, hp, stride=d - 1) == B.SM_EINVAL
    assert _step(L, mats, hp, stride=words) == B.SM_EINVAL
    same_words = [mats[0], (96, 64, mats[1][2], 0)]          # word_off ignored
    assert _step(L, same_words, hp, stride=d, ws_bytes=1024) == B.SM_EWORKSPACE
    c = hp.to_c()
    c.sign_encoding = 2
    arr = B.mats_array(mats)
    assert L.signmuon_step(arr, len(mats), ctypes.byref(c), FAKE, FAKE, 1, FAKE, FAKE, d, 3,
                           0, 0, None, FAKE, 1 << 30, None, None) == B.SM_EINVAL
    assert B.step_workspace(mats, hp, 0) > 0
    # int8 and packed signs both come straight from the last epilogue (no
    # float32 U is kept for any width)
    m1, _, _ = B.default_layout([(5, 37)])
    assert B.step_workspace(m1, hp, 0) == B.step_workspace(m1, _hp(), 0) > 0


def test_step_normalized_validation():
    # the normalized sign step needs P >= 1 power steps whatever the scale,
    # and keeps the raw Gram and power vectors in its workspace
    L = B.lib()
    mats, d, words = B.default_layout([(64, 96), (96, 64)])
    assert _step(L, mats, _hp(P=0), post=3) == B.SM_EINVAL
    assert _step(L, mats, _hp(P=300), post=3) == B.SM_EINVAL
    assert B.step_workspace(mats, _hp(P=0), 3) == 0
    assert B.step_workspace(mats, _hp(P=5), 3) > B.step_workspace(mats, _hp(P=5), 0)
    assert B.step_workspace(mats, _hp(P=5), 4) == 0
