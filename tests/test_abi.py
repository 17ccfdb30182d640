"""Host-side checks of the C-ABI library (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:int|void|size_t|const char)\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("moe_layer_create", "moe_load_expert", "moe_forward", "moe_map_expert",
                 "moe_status", "moe_destroy"):
        assert must in names


def test_library_exports_every_declared_symbol():
    from int4_weight_expert_amd import moe as M
    lib = ctypes.CDLL(M.LIB_PATH)
    names = declared_functions()
    assert set(names) == set(M.EXPORTS), set(names) ^ set(M.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    M.lib()          # the binding's signatures resolve against the library


def test_null_arguments_are_rejected_without_device_work():
    from int4_weight_expert_amd import moe as M
    L = M.lib()
    assert L.moe_forward(None, None, 1, 0, None) == M.MOE_E_ARG
    assert L.moe_expert_bytes(None) == 0
    assert L.moe_map_expert(None, 0, 0, 0) == M.MOE_E_ARG
    assert L.moe_pack_int4_rows(None, 1, 2, None, None, None) == M.MOE_E_ARG
    assert L.moe_bucket(None, 1, 1, 1, None, None, None, None, None, None) == M.MOE_E_ARG
    L.moe_destroy(None)


def test_create_rejects_unsupported_config_before_touching_a_device():
    from int4_weight_expert_amd import moe as M
    # invalid router groupings: groups not dividing E, one-expert groups,
    # more groups kept than exist, K above the kept experts
    bad = [dict(n_group=3, topk_group=1), dict(n_group=32, topk_group=4),
           dict(n_group=8, topk_group=9), dict(n_group=16, topk_group=1),
           dict(E=300), dict(K=9), dict(H=6000), dict(wfmt=3), dict(max_tokens=0)]
    for kw in bad:
        base = dict(H=512, I=256, E=32, K=4, n_shared=1, n_layers=1, wfmt=1, n_slots=32,
                    max_tokens=4)
        ng, tg = kw.pop("n_group", 1), kw.pop("topk_group", 1)
        base.update(kw)
        cfg = M.make_config(base["H"], base["I"], base["E"], base["K"], base["n_shared"],
                            base["n_layers"], base["wfmt"], base["n_slots"], base["max_tokens"],
                            n_group=ng, topk_group=tg)
        rc, h = M.moe_layer_create_rc(cfg)
        assert rc in (M.MOE_E_ARG, M.MOE_E_UNSUPPORTED), (kw, rc)
        assert not h


def test_no_cpu_fallback_without_a_gpu():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from int4_weight_expert_amd import moe as M
    cfg = M.make_config(512, 256, 32, 4, 1, 1, 1, 32, 4)
    rc, h = M.moe_layer_create_rc(cfg)
    assert rc == M.MOE_E_HIP and not h


def test_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "int4_weight_expert_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "moe_oracle" not in txt, f


def test_every_status_code_has_a_producing_path():
    """Each MOE_E_* code the header defines is returned by some path of the
    library source (the GPU tests produce each one at run time; MOE_E_HIP
    is produced here, without a GPU, by create)."""
    hdr = open(HEADER, encoding="utf-8").read()
    codes = re.findall(r"#define\s+(MOE_E_\w+)\s", hdr)
    assert len(codes) >= 9
    csrc = os.path.join(ROOT, "int4_weight_expert_amd", "csrc")
    src = "".join(open(os.path.join(csrc, f), encoding="utf-8").read()
                  for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    for code in codes:
        produced = re.search(r"(return|\?|:)\s*" + code + r"\b", src)
        assert produced, f"{code} is never returned"
    # the device-side codes are raised by a status bit that a kernel sets
    assert "atomicOr(&f.status[0], (uint32_t)STATUS_RANGE)" in src
    assert "atomicOr(&f.status[0], (uint32_t)STATUS_NOT_RESIDENT)" in src
