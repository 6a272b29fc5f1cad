"""The C-ABI library without a GPU: it loads, exports every function that
include/nvq.h declares, and its host-side logic (status strings, argument
and size validation, workspace sizing, the GEMM grid setting) behaves as the
header states. No call here launches a kernel."""
import ctypes as C
import os
import re

import precision_moe_numerics_amd as nvq

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "nvq.h")

NVQ_OK, NVQ_ERR_NULL, NVQ_ERR_DIM, NVQ_ERR_WORKSPACE = 0, -1, -2, -3
NVQ_ERR_LAUNCH, NVQ_ERR_UNSUPPORTED, NVQ_ERR_ALIGN = -4, -5, -6


def declared_functions():
    """Names of the functions the header declares (comments, preprocessor
    lines, enums and typedefs removed; what remains are prototypes)."""
    s = open(HEADER).read()
    s = re.sub(r"/\*.*?\*/", "", s, flags=re.S)
    s = re.sub(r"//[^\n]*", "", s)
    s = re.sub(r"#[^\n]*", "", s)
    s = re.sub(r"typedef\s+struct\s*\{.*?\}\s*\w+\s*;", "", s, flags=re.S)
    s = re.sub(r"enum\s*\{.*?\}\s*;", "", s, flags=re.S)
    s = re.sub(r"typedef[^;]*;", "", s)
    return re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}]*\)\s*;", s)


def test_header_parse_finds_the_api():
    names = declared_functions()
    assert len(names) == len(set(names))
    for must in ("nvfp4_quantize", "moe_expert_fwd_nvfp4", "moe_fc1_swiglu_nvfp4", "moe_fc2_nvfp4",
                 "mxfp8_requant_sr", "moe_grouped_gemm_mxfp8", "swiglu_bwd", "rht32_blockquant",
                 "rht32_dequant_combine", "nvq_set_gemm_workgroups"):
        assert must in names


def test_library_exports_every_declared_function():
    L = nvq.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, f"declared in nvq.h but not exported: {missing}"


def test_status_strings_and_version():
    L = nvq.lib()
    assert L.nvq_abi_version() >= 1
    texts = set()
    for code in (NVQ_OK, NVQ_ERR_NULL, NVQ_ERR_DIM, NVQ_ERR_WORKSPACE, NVQ_ERR_LAUNCH, NVQ_ERR_UNSUPPORTED,
                 NVQ_ERR_ALIGN):
        t = L.nvq_status_string(code)
        assert t and len(t) > 0
        texts.add(t)
    assert len(texts) == 7  # one distinct message per status


def test_gemm_workgroups_range():
    L = nvq.lib()
    assert L.nvq_set_gemm_workgroups(-1) == NVQ_ERR_DIM
    assert L.nvq_set_gemm_workgroups(1025) == NVQ_ERR_DIM
    assert L.nvq_set_gemm_workgroups(1024) == NVQ_OK
    assert L.nvq_set_gemm_workgroups(0) == NVQ_OK


def test_workspace_sizes_grow_with_the_problem():
    L = nvq.lib()
    small = L.moe_expert_fwd_nvfp4_workspace_size(64, 256, 2, 4, 256)
    large = L.moe_expert_fwd_nvfp4_workspace_size(4096, 256, 2, 4, 256)
    assert 0 < small < large
    assert 0 < L.moe_fc1_workspace_size(100, 8) <= L.moe_fc1_workspace_size(100000, 8)
    assert L.moe_fc2_workspace_size(100, 8) == L.moe_fc1_workspace_size(100, 8)


def _fake(n=1):
    """Distinct non-null, 256-byte aligned addresses that are never dereferenced:
    every call below is rejected by the host checks before any device work."""
    return [C.c_void_p(0x100000 + 0x1000 * i) for i in range(n)]


def _fwd(L, T=64, d=256, k=2, E=4, d_ff=256, null_x=False, ws_bytes=1 << 30):
    p = _fake(11)
    x = None if null_x else p[0]
    return L.moe_expert_fwd_nvfp4(x, T, d, p[1], k, E, d_ff, p[2], p[3], p[4], p[5], p[6], p[7], p[8], None,
                                  p[9], ws_bytes, None)


def test_forward_argument_checks():
    L = nvq.lib()
    assert _fwd(L, null_x=True) == NVQ_ERR_NULL
    assert _fwd(L, d=200) == NVQ_ERR_DIM           # d not a multiple of 128
    assert _fwd(L, d_ff=100) == NVQ_ERR_DIM        # d_ff not a multiple of 128
    assert _fwd(L, k=5, E=4) == NVQ_ERR_DIM        # k > E
    assert _fwd(L, E=5000, k=2) == NVQ_ERR_DIM     # E above 4096
    assert _fwd(L, T=1 << 22, d=4096) == NVQ_ERR_DIM  # T*d/2 codes past 32-bit offsets
    assert _fwd(L, d=65536, d_ff=65536) == NVQ_ERR_DIM  # d*d_ff past 32-bit weight offsets
    need = L.moe_expert_fwd_nvfp4_workspace_size(64, 256, 2, 4, 256)
    assert _fwd(L, ws_bytes=need - 1) == NVQ_ERR_WORKSPACE
