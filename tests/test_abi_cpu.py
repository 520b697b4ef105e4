"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, reports workspace sizes, and rejects invalid arguments on the
host before anything is enqueued (every call here fails validation, so no
kernel is ever launched)."""
import ctypes
import os
import re

import pytest

from precision_moe_expert_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_lp.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", src, re.M)))


def test_header_declares_expected_entry_points():
    fns = declared_functions()
    for name in ("moe_route_permute", "moe_expert_forward", "moe_combine", "moe_workspace_bytes",
                 "moe_lm_head_logprob", "moe_status_str", "moe_abi_version", "moe_expert_forward_materialized",
                 "moe_materialized_workspace_bytes", "moe_pack_weights_kblocked"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.moe_abi_version() == 6


def test_status_strings():
    for s in range(5):
        assert binding.status_str(s)
    assert binding.status_str(99) == "unknown status"


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "moe_lp.h"\nint main(void){ moe_layer l; (void)l; return MOE_OK; }\n')
    import subprocess
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c", str(src),
                           "-o", str(tmp_path / "t.o")])


def test_workspace_sizes():
    L = binding.make_layer(4096, 2048, 768, 128, 8, binding.FMT_FP8)
    n = binding.workspace_bytes(L, 16)
    R = 4096 * 8
    assert n >= R * 2048 * 2 + R * 768 + 4096 * 2048  # y + h + x codes
    assert binding.workspace_bytes(L, 1) == n          # independent of the chunk size
    assert binding.workspace_bytes(binding.make_layer(4096, 2048, 768, 128, 8, 9), 16) == 0
    # LM head: (max, sum of exponentials) per token and 128-row vocabulary block, then the target logits
    assert binding.lib().moe_lm_head_workspace_bytes(64, 32000) == 64 * 250 * 2 * 4 + 256


FAKE = 1 << 20  # aligned non-null address; never dereferenced because validation fails first


def _fwd(layer, x=FAKE, lg=FAKE, w=FAKE, adapter=None, chunk=1, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    qw = binding.MoeQWeights(w, w)
    sc = binding.MoeScales(w, w, None, None)
    return binding.lib().moe_expert_forward(ctypes.byref(layer), x, lg, ctypes.byref(qw), ctypes.byref(sc), adapter,
                                            chunk, out, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    (dict(H=200), binding.MOE_ERR_UNSUPPORTED),
    (dict(I=100), binding.MOE_ERR_UNSUPPORTED),
    (dict(I=384), None),
    (dict(I=384, fmt=2), None),
    (dict(E=2000), binding.MOE_ERR_UNSUPPORTED),
    (dict(k=17, E=32), binding.MOE_ERR_UNSUPPORTED),
    (dict(k=9, E=8), binding.MOE_ERR_INVALID_ARGUMENT),
    (dict(k=0), binding.MOE_ERR_INVALID_ARGUMENT),
    (dict(T=-1), binding.MOE_ERR_INVALID_ARGUMENT),
    (dict(fmt=7), binding.MOE_ERR_INVALID_ARGUMENT),
])
def test_forward_rejects_bad_layer(case, expect):
    p = dict(T=64, H=256, I=512, E=8, k=2, fmt=1)
    p.update(case)
    L = binding.make_layer(p["T"], p["H"], p["I"], p["E"], p["k"], p["fmt"])
    if expect is None:  # a valid layer: validation passes and the fake workspace size is what fails
        assert _fwd(L, ws_bytes=0) == binding.MOE_ERR_WORKSPACE_TOO_SMALL
    else:
        assert _fwd(L) == expect


def test_nvfp4_host_checks():
    """NVFP4: forward workspace as for INT4 (16-bit activations); the
    second-level scale pointers are required, with or without an adapter.  Backward: the transposed copy holds one fp16 per E4M3
    scale (16 weights); its workspace is INT4's."""
    Ln = binding.make_layer(64, 256, 512, 8, 2, binding.FMT_NVFP4)
    Li = binding.make_layer(64, 256, 512, 8, 2, binding.FMT_INT4)
    assert binding.workspace_bytes(Ln, 4) == binding.workspace_bytes(Li, 4) > 0
    lib = binding.lib()

    def fwd(g13, g2, ws_bytes=0):
        qw = binding.MoeQWeights(FAKE, FAKE)
        sc = binding.MoeScales(FAKE, FAKE, g13, g2)
        return lib.moe_expert_forward(ctypes.byref(Ln), FAKE, FAKE, ctypes.byref(qw), ctypes.byref(sc), None, 1,
                                      FAKE, FAKE, ws_bytes, None)
    assert fwd(None, FAKE) == binding.MOE_ERR_INVALID_ARGUMENT
    assert fwd(FAKE, FAKE + 2) == binding.MOE_ERR_INVALID_ARGUMENT           # misaligned fp32
    assert fwd(FAKE, FAKE + 4) == binding.MOE_ERR_WORKSPACE_TOO_SMALL        # valid; the workspace fails
    Lo = binding.make_layer(64, 256, 512, 8, 2, binding.FMT_NVFP4, oft=True)
    assert _fwd(Lo, adapter=FAKE) == binding.MOE_ERR_INVALID_ARGUMENT     # adapter accepted; no g13 / g2
    assert binding.materialized_workspace_bytes(Ln, 4) == binding.materialized_workspace_bytes(Li, 4) > 0
    assert _mat(Ln) == binding.MOE_ERR_INVALID_ARGUMENT                     # no second-level scales
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    E, H, I = 8, 256, 512
    assert binding.backward_weights_bytes(Ln) == (al(E * H * I) + al(E * I * H // 2) + al(E * (H // 16) * 2 * I * 2)
                                                  + al(E * (I // 16) * H * 2))
    assert binding.backward_workspace_bytes(Ln, 4) == binding.backward_workspace_bytes(Li, 4) > 0
    qw = binding.MoeQWeights(FAKE, FAKE)
    for g13, g2 in ((None, FAKE), (FAKE, FAKE + 2)):
        sc = binding.MoeScales(FAKE, FAKE, g13, g2)
        assert lib.moe_expert_backward(ctypes.byref(Ln), FAKE, FAKE, ctypes.byref(qw), ctypes.byref(sc), FAKE, None,
                                       FAKE, 1, FAKE, FAKE, None, FAKE, 1 << 40, None, None,
                                       None) == binding.MOE_ERR_INVALID_ARGUMENT


def test_forward_rejects_bad_pointers_and_workspace():
    L = binding.make_layer(64, 256, 512, 8, 2, 1)
    assert _fwd(L, x=None) == binding.MOE_ERR_INVALID_ARGUMENT
    assert _fwd(L, out=FAKE + 4) == binding.MOE_ERR_INVALID_ARGUMENT       # misaligned
    assert _fwd(L, chunk=0) == binding.MOE_ERR_INVALID_ARGUMENT
    assert _fwd(L, adapter=FAKE) == binding.MOE_ERR_INVALID_ARGUMENT       # adapter without oft_block
    assert _fwd(L, ws_bytes=1000) == binding.MOE_ERR_WORKSPACE_TOO_SMALL
    Lo = binding.make_layer(64, 256, 512, 8, 2, 1, oft=True)
    assert _fwd(Lo) == binding.MOE_ERR_INVALID_ARGUMENT                    # oft_block without adapter
    Lf = binding.make_layer(64, 256, 512, 8, 2, binding.FMT_FP8, oft=True)
    assert _fwd(Lf, adapter=FAKE + 2) == binding.MOE_ERR_INVALID_ARGUMENT  # misaligned adapter
    assert _fwd(Lf, adapter=FAKE, ws_bytes=1000) == binding.MOE_ERR_WORKSPACE_TOO_SMALL  # OFT on FP8 accepted
    L0 = binding.make_layer(0, 256, 512, 8, 2, 1)
    assert _fwd(L0, x=None, lg=None, w=None, out=None, ws=None) == binding.MOE_OK  # T = 0: no-op


def test_other_entry_points_reject_bad_args():
    L = binding.make_layer(64, 256, 512, 8, 2, 1)
    lib = binding.lib()
    assert lib.moe_combine(ctypes.byref(L), None, FAKE, FAKE, FAKE, None) == binding.MOE_ERR_INVALID_ARGUMENT
    ro = binding.MoeRouteOut(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE)
    assert lib.moe_route_permute(ctypes.byref(L), FAKE, ctypes.byref(ro), FAKE, 1 << 30, None) == \
        binding.MOE_ERR_INVALID_ARGUMENT
    ro = binding.MoeRouteOut(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert lib.moe_route_permute(ctypes.byref(L), FAKE, ctypes.byref(ro), FAKE, 8, None) == \
        binding.MOE_ERR_WORKSPACE_TOO_SMALL
    assert lib.moe_lm_head_logprob(4, 100, 10, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == \
        binding.MOE_ERR_UNSUPPORTED
    assert lib.moe_lm_head_logprob(4, 128, 10, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None) == \
        binding.MOE_ERR_WORKSPACE_TOO_SMALL


def _mat(layer, chunk=1, ws_bytes=1 << 40, ms=None, n=None, x=FAKE):
    qw = binding.MoeQWeights(FAKE, FAKE)
    sc = binding.MoeScales(FAKE, FAKE, None, None)
    return binding.lib().moe_expert_forward_materialized(ctypes.byref(layer), x, FAKE, ctypes.byref(qw),
                                                         ctypes.byref(sc), None, chunk, FAKE, FAKE, ws_bytes, None,
                                                         ms, n)


def test_materialized_workspace_grows_with_the_chunk():
    H, I, E = 7168, 2048, 384
    L = binding.make_layer(8192, H, I, E, 8, binding.FMT_INT4)
    sizes = {c: binding.materialized_workspace_bytes(L, c) for c in (1, 8, 32, 64)}
    for a, b in ((1, 8), (8, 32), (32, 64)):
        # exactly (b - a) more experts' BF16 copies, up to alignment
        assert abs(sizes[b] - sizes[a] - (b - a) * 3 * H * I * 2) <= 256
    assert binding.materialized_workspace_bytes(L, 10 ** 6) == binding.materialized_workspace_bytes(L, E)
    assert binding.materialized_workspace_bytes(L, 0) == 0


def test_materialized_rejects_bad_args():
    L = binding.make_layer(64, 256, 512, 8, 2, 1)
    ms = (ctypes.c_float * len(binding.STAGES))()
    n = (ctypes.c_int32 * len(binding.STAGES))()
    assert _mat(L, chunk=0) == binding.MOE_ERR_INVALID_ARGUMENT
    assert _mat(L, x=None) == binding.MOE_ERR_INVALID_ARGUMENT
    assert _mat(L, ms=ms) == binding.MOE_ERR_INVALID_ARGUMENT              # one timing array without the other
    assert _mat(L, ws_bytes=binding.materialized_workspace_bytes(L, 2) - 1, chunk=2) == \
        binding.MOE_ERR_WORKSPACE_TOO_SMALL
    assert _mat(L, ws_bytes=0, ms=ms, n=n) == binding.MOE_ERR_WORKSPACE_TOO_SMALL


def test_kblocked_layout_host_checks():
    """The 16 x 128 tiled code layout: fused forward, materialized forward and
    backward take it with the same workspace sizes as rows; an unknown layout
    value is invalid; the pack entry rejects bad pointers."""
    lib = binding.lib()
    Lk = binding.make_layer(64, 256, 512, 8, 2, binding.FMT_INT4, weight_layout=binding.WL_KBLOCKED)
    Lr = binding.make_layer(64, 256, 512, 8, 2, binding.FMT_INT4)
    assert binding.workspace_bytes(Lk, 4) == binding.workspace_bytes(Lr, 4) > 0
    assert _fwd(Lk, ws_bytes=0) == binding.MOE_ERR_WORKSPACE_TOO_SMALL      # accepted up to the workspace check
    bad = binding.make_layer(64, 256, 512, 8, 2, binding.FMT_INT4, weight_layout=2)
    assert binding.workspace_bytes(bad, 4) == 0
    assert _fwd(bad) == binding.MOE_ERR_INVALID_ARGUMENT
    for fmt in (binding.FMT_FP8, binding.FMT_FP8_POW2, binding.FMT_MXFP4):
        Lf = binding.make_layer(64, 256, 512, 8, 2, fmt, weight_layout=binding.WL_KBLOCKED)
        assert _fwd(Lf, ws_bytes=0) == binding.MOE_ERR_WORKSPACE_TOO_SMALL
        Lfr = binding.make_layer(64, 256, 512, 8, 2, fmt)
        assert binding.materialized_workspace_bytes(Lf, 4) == binding.materialized_workspace_bytes(Lfr, 4) > 0
        assert binding.backward_weights_bytes(Lf) > 0
    assert binding.materialized_workspace_bytes(Lk, 4) == binding.materialized_workspace_bytes(Lr, 4) > 0
    assert _mat(Lk, ws_bytes=0) == binding.MOE_ERR_WORKSPACE_TOO_SMALL
    assert binding.backward_weights_bytes(Lk) == binding.backward_weights_bytes(Lr) > 0
    assert binding.backward_workspace_bytes(Lk, 4) == binding.backward_workspace_bytes(Lr, 4) > 0
    qw = binding.MoeQWeights(FAKE, FAKE)
    pack = lambda L, o13=FAKE, o2=FAKE: lib.moe_pack_weights_kblocked(ctypes.byref(L), ctypes.byref(qw), o13, o2,
                                                                       None)  # noqa: E731
    assert pack(Lr, o13=None) == binding.MOE_ERR_INVALID_ARGUMENT
    assert pack(Lr, o2=FAKE + 8) == binding.MOE_ERR_INVALID_ARGUMENT
    assert pack(bad) == binding.MOE_ERR_INVALID_ARGUMENT
