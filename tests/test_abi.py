"""The C ABI without a GPU: the library loads, exports every entry point that
include/ddtree.h declares, and rejects invalid host arguments with the
documented status codes before touching the device."""
import ctypes
import re
from pathlib import Path

import pytest

from tree_verify_mla_amd import _lib

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "ddtree.h"

EINVAL, EUNSUPPORTED, EWORKSPACE = -1, -2, -3
NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddtree_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_stages():
    names = declared_functions()
    for n in ("ddtree_build_tree", "ddtree_compile_visibility", "ddtree_verify_attn", "ddtree_accept",
              "ddtree_commit_kv", "ddtree_drafter_topk", "ddtree_tree_sample",
              "ddtree_verify_attn_layers"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} missing from libddtree.so"


def test_abi_version(lib):
    assert lib.ddtree_abi_version() == 1


def _err(lib):
    return lib.ddtree_last_error().decode()


def test_build_tree_validation(lib):
    f = lib.ddtree_build_tree
    assert f(FAKE, FAKE, FAKE, FAKE, -1, 7, 4, 8, FAKE, FAKE, FAKE, NULL, NULL) == EINVAL
    assert f(FAKE, FAKE, NULL, FAKE, 1, 7, 4, 8, FAKE, FAKE, FAKE, NULL, NULL) == EINVAL
    # 1 + 1 = 2 rank paths reachable with depth 2, top-1
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 3, FAKE, FAKE, FAKE, NULL, NULL) == EINVAL
    assert "reachable" in _err(lib)
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 0, 4, 3, FAKE, FAKE, FAKE, NULL, NULL) == EINVAL
    # rank paths must pack into 64 bits: depth 20 x 8 bits (top-256) does not
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 20, 256, 8, FAKE, FAKE, FAKE, NULL, NULL) == EUNSUPPORTED
    assert f(NULL, NULL, NULL, NULL, 0, 7, 4, 8, NULL, NULL, NULL, NULL, NULL) == 0  # empty batch


def test_visibility_validation(lib):
    f = lib.ddtree_compile_visibility
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 33, 1, FAKE, NULL, NULL, NULL, NULL) == EINVAL  # W too small
    assert "words_per_row" in _err(lib)
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 33, 2, FAKE, NULL, FAKE, NULL, NULL) == EINVAL  # mask w/o indptr
    assert f(NULL, FAKE, FAKE, FAKE, 2, 33, 2, FAKE, NULL, NULL, NULL, NULL) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 0, 2, FAKE, NULL, NULL, NULL, NULL) == EINVAL


def _attn(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, num_slots=100, kvp=FAKE, kvi=FAKE, qo=FAKE, vis=FAKE, W=2, bs=1, H=8,
             max_q=33, max_kv=100, scale=0.14468, dtype=_lib.DDTREE_F32, out=FAKE, lse=NULL,
             splits=1, ws=NULL, ws_bytes=0)
    a.update(kw)
    return lib.ddtree_verify_attn(a["q"], a["kv"], a["num_slots"], a["kvp"], a["kvi"], a["qo"],
                                  a["vis"], a["W"], a["bs"], a["H"], a["max_q"], a["max_kv"],
                                  a["scale"], a["dtype"], a["out"], a["lse"], a["splits"], a["ws"],
                                  a["ws_bytes"], NULL)


def test_verify_attn_validation(lib):
    assert _attn(lib, bs=-1) == EINVAL
    assert _attn(lib, q=NULL) == EINVAL
    assert _attn(lib, H=0) == EINVAL
    assert _attn(lib, max_kv=10) == EINVAL          # max_kv_len < max_q_len
    assert _attn(lib, W=1) == EINVAL                # 32 bits cannot cover 33 nodes
    assert _attn(lib, scale=float("nan")) == EINVAL
    assert _attn(lib, num_slots=0) == EINVAL
    assert _attn(lib, splits=-1) == EINVAL
    assert _attn(lib, dtype=7) == EINVAL
    assert _attn(lib, splits=4, ws=NULL, ws_bytes=0) == EWORKSPACE
    assert "workspace" in _err(lib)
    assert _attn(lib, bs=0) == 0


def test_workspace_size_forced_split(lib):
    # fp32 tiles hold 4 rows; 33 nodes x 8 heads = 264 rows -> 66 tiles
    per_slot = 4 * (512 + 2) * 4
    assert lib.ddtree_verify_attn_workspace_size(2, 8, 33, 100, 3, _lib.DDTREE_F32) == 2 * 66 * 3 * per_slot
    assert lib.ddtree_verify_attn_workspace_size(2, 8, 33, 100, 1, _lib.DDTREE_F32) == 0
    assert lib.ddtree_verify_attn_workspace_size(2, 8, 33, 100, 0, _lib.DDTREE_F32) == 0
    # bf16 tiles hold 128 rows -> 3 tiles
    # bf16: per slot O / l of 128 rows x 512 in fp16, then m, l and four
    # quarter scales per row in fp32
    assert lib.ddtree_verify_attn_workspace_size(1, 8, 33, 100, 2, _lib.DDTREE_BF16) == 3 * 2 * 128 * (256 + 6) * 4
    assert lib.ddtree_verify_attn_workspace_size(-1, 8, 33, 100, 2, _lib.DDTREE_BF16) == 0


def test_verify_attn_plan_validation(lib):
    rows, splits = ctypes.c_int(-7), ctypes.c_int(-7)
    out = (ctypes.byref(rows), ctypes.byref(splits))
    assert lib.ddtree_verify_attn_plan(1, 8, 33, 4129, 0, _lib.DDTREE_BF16, NULL, out[1]) == EINVAL
    assert lib.ddtree_verify_attn_plan(1, 0, 33, 4129, 0, _lib.DDTREE_BF16, *out) == EINVAL
    assert lib.ddtree_verify_attn_plan(1, 8, 33, 32, 0, _lib.DDTREE_BF16, *out) == EINVAL
    assert lib.ddtree_verify_attn_plan(1, 8, 33, 4129, -1, _lib.DDTREE_BF16, *out) == EINVAL
    assert lib.ddtree_verify_attn_plan(1, 8, 33, 4129, 0, 7, *out) == EINVAL
    # the fp32 kernel needs no device to plan: 4-row tiles, one part unless forced
    assert lib.ddtree_verify_attn_plan(1, 8, 33, 4129, 0, _lib.DDTREE_F32, *out) == 0
    assert (rows.value, splits.value) == (4, 1)
    assert lib.ddtree_verify_attn_plan(1, 8, 33, 4129, 3, _lib.DDTREE_F32, *out) == 0
    assert (rows.value, splits.value) == (4, 3)


def test_accept_validation(lib):
    f = lib.ddtree_accept
    assert f(FAKE, FAKE, FAKE, FAKE, -1, 7, FAKE, FAKE, FAKE, FAKE, NULL) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, -1, FAKE, FAKE, FAKE, FAKE, NULL) == EINVAL
    assert f(FAKE, NULL, FAKE, FAKE, 1, 7, FAKE, FAKE, FAKE, FAKE, NULL) == EINVAL
    assert f(NULL, NULL, NULL, NULL, 0, 7, NULL, NULL, NULL, NULL, NULL) == 0


def test_commit_kv_validation(lib):
    f = lib.ddtree_commit_kv
    args = dict(kvp=FAKE, kvi=FAKE, qo=FAKE, nodes=FAKE, alen=FAKE, bs=1, D=7, maxkv=100, nkvp=FAKE,
                nkvi=FAKE, cap=100, pool=NULL, nslots=0, dtype=_lib.DDTREE_BF16, stream=NULL)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())
    assert call(bs=-1) == EINVAL
    assert call(kvi=NULL) == EINVAL
    assert call(nkvp=NULL) == EINVAL
    assert call(D=-1) == EINVAL
    assert call(maxkv=0) == EINVAL
    assert call(cap=-1) == EINVAL
    assert call(pool=FAKE, nslots=0) == EINVAL          # a pool needs slots
    assert call(pool=FAKE, nslots=10, dtype=7) == EINVAL
    assert call(maxkv=2**31 - 1) == EUNSUPPORTED        # more than 65535 prefix chunks
    assert "commit_kv" in _err(lib)
    assert call(bs=0, kvp=NULL, kvi=NULL, qo=NULL, nodes=NULL, alen=NULL, nkvp=NULL, nkvi=NULL) == 0


def test_drafter_topk_validation(lib):
    f = lib.ddtree_drafter_topk
    F32 = _lib.DDTREE_F32
    assert f(FAKE, F32, -1, 100, 8, FAKE, FAKE, FAKE, 1 << 20, NULL) == EINVAL
    assert f(NULL, F32, 4, 100, 8, FAKE, FAKE, FAKE, 1 << 20, NULL) == EINVAL
    assert f(FAKE, 9, 4, 100, 8, FAKE, FAKE, FAKE, 1 << 20, NULL) == EINVAL
    assert f(FAKE, F32, 4, 100, 0, FAKE, FAKE, FAKE, 1 << 20, NULL) == EINVAL
    assert f(FAKE, F32, 4, 5, 8, FAKE, FAKE, FAKE, 1 << 20, NULL) == EINVAL      # topk > vocab
    assert f(FAKE, F32, 4, 100, 33, FAKE, FAKE, FAKE, 1 << 20, NULL) == EUNSUPPORTED
    assert f(FAKE, F32, 4, 8192 * 200, 8, FAKE, FAKE, FAKE, 1 << 30, NULL) == EUNSUPPORTED
    need = lib.ddtree_drafter_topk_workspace_size(4, 100, 8)
    assert need == 4 * 1 * (2 + 16) * 4
    assert lib.ddtree_drafter_topk_workspace_size(2, 8193, 3) == 2 * 2 * (2 + 6) * 4
    assert f(FAKE, F32, 4, 100, 8, FAKE, FAKE, FAKE, need - 1, NULL) == EWORKSPACE
    assert f(FAKE, F32, 4, 100, 8, FAKE, FAKE, NULL, need, NULL) == EWORKSPACE
    assert "drafter_topk" in _err(lib)
    assert f(NULL, F32, 0, 100, 8, NULL, NULL, NULL, 0, NULL) == 0


def test_tree_sample_validation(lib):
    f = lib.ddtree_tree_sample
    ws = lib.ddtree_tree_sample_workspace_size(33)
    assert ws == 33 * 256 * 8 and lib.ddtree_tree_sample_workspace_size(0) == 0
    args = [FAKE] * 6 + [1, 33, 7, 512] + [FAKE] * 5 + [ws, NULL]
    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(6, -1) == EINVAL        # bs
    assert call(3, NULL) == EINVAL      # target_probs
    assert call(7, -1) == EINVAL        # total_q
    assert call(8, -1) == EINVAL        # depth_max
    assert call(9, 0) == EINVAL         # vocab
    assert "tree_sample" in _err(lib)
    assert call(9, 256 * 8192 + 1) == EUNSUPPORTED
    assert call(15, ws - 1) == EWORKSPACE
    assert call(14, NULL) == EWORKSPACE
    assert "workspace" in _err(lib)
    assert f(*([NULL] * 6 + [0, 0, 7, 512] + [NULL] * 5 + [0, NULL])) == 0


def test_binding_rejects_host_tensors():
    import torch
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        _lib.ddtree_accept(t, t, t, t, 7, t, t, t, t)


def test_verify_attn_layers_validation(lib):
    f = lib.ddtree_verify_attn_layers
    F32 = _lib.DDTREE_F32
    # L, q, q_ls, kv, kv_ls, num_slots, kvp, kvi, qo, vis, W, bs, H, max_q, max_kv, scale, dtype,
    # out, out_ls, lse, lse_ls, splits, ws, ws_bytes, stream
    args = [2, FAKE, 100, FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 9, 20, 0.1, F32,
            FAKE, 100, NULL, 0, 0, NULL, 0, NULL]
    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(0, 0) == EINVAL and "num_layers" in _err(lib)
    assert call(0, 65536) == EINVAL
    assert call(2, -1) == EINVAL and "stride" in _err(lib)
    assert call(4, -1) == EINVAL
    assert call(18, -5) == EINVAL
    assert call(1, NULL) == EINVAL
    assert call(16, 7) == EINVAL                       # dtype
    assert call(18, 0) == EINVAL and "overlap" in _err(lib)   # layers writing one output
    a = list(args)
    a[19], a[20] = FAKE, 0                             # lse given with a zero stride
    assert f(*a) == EINVAL
    a = list(args)
    a[0], a[18] = 1, 0                                 # one layer: stride unused
    assert f(*a) != EINVAL or "overlap" not in _err(lib)
    # workspace: L single-layer workspaces
    one = lib.ddtree_verify_attn_workspace_size(2, 8, 33, 100, 3, F32)
    assert lib.ddtree_verify_attn_layers_workspace_size(5, 2, 8, 33, 100, 3, F32) == 5 * one
    assert lib.ddtree_verify_attn_layers_workspace_size(0, 2, 8, 33, 100, 3, F32) == 0
    a = list(args)
    a[21], a[23] = 3, 2 * lib.ddtree_verify_attn_workspace_size(1, 8, 9, 20, 3, F32) - 1
    a[22] = FAKE
    assert f(*a) == EWORKSPACE
    a = list(args)
    a[11] = 0                                          # bs == 0: nothing to do
    assert f(*a) == 0


def test_validate_inputs_host_checks(lib):
    f = lib.ddtree_validate_inputs
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert f(1, FAKE, 10, FAKE, FAKE, 10, 10, NULL, NULL, NULL, NULL) == EINVAL     # no report
    assert "report" in _err(lib)
    assert f(-1, FAKE, 10, FAKE, FAKE, 10, 10, NULL, NULL, FAKE, NULL) == EINVAL
    assert f(1, NULL, 10, FAKE, FAKE, 10, 10, NULL, NULL, FAKE, NULL) == EINVAL
    assert f(1, FAKE, 10, FAKE, NULL, 10, 10, NULL, NULL, FAKE, NULL) == EINVAL
    assert f(70000, FAKE, 10, FAKE, FAKE, 10, 10, NULL, NULL, FAKE, NULL) == EUNSUPPORTED


def test_build_tree_visibility_validation(lib):
    f = lib.ddtree_build_tree_visibility
    # lp, ids, roots, qo, prefix, bs, D, K, max_budget, max_q, W, tok, par, dep, sc, bits, pos, stream
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 7, 8, 32, 33, 2, FAKE, FAKE, FAKE, NULL, FAKE, NULL, NULL]
    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(5, -1) == EINVAL
    assert call(2, NULL) == EINVAL                  # root tokens
    a = list(args)
    a[6], a[7], a[8] = 2, 2, 7                      # 2 + 4 rank paths cannot hold 7 nodes
    assert f(*a) == EINVAL and "reachable" in _err(lib)
    assert call(8, 4096) == EUNSUPPORTED            # above 2048
    assert call(10, 1) == EINVAL and "words_per_row" in _err(lib)
    assert call(15, NULL) == EINVAL                 # vis_bits
    a = list(args)
    a[16], a[4] = FAKE, NULL                        # positions without prefix_lens
    assert f(*a) == EINVAL
    assert call(9, 0) == EINVAL                     # max_q_len
    assert call(5, 0) == 0                          # empty batch


def test_measurement_probes_reject_bad_arguments(lib):
    f = lib.ddtree_probe_mfma_loop
    assert f(0, 1, FAKE, NULL) == EINVAL
    assert f(1, 0, FAKE, NULL) == EINVAL
    assert f(1, 1, NULL, NULL) == EINVAL
    assert "probe_mfma_loop" in _err(lib)
    assert lib.ddtree_device_info(NULL, NULL) == EINVAL
