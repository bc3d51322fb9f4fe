"""ctypes binding of libddtree.so (declared in include/ddtree.h).

Argument marshalling only: every function checks that the tensors it is
handed are contiguous device tensors of the expected dtype, passes their
device pointers and the current torch stream to the C entry point of the
same name, and raises ``DDTreeError`` on a non-zero status.  All arithmetic
happens in the library's HIP kernels; outputs are written into the tensors
the caller provides.  There is no fallback: if the library is missing,
loading raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

import torch

LIB_PATH = Path(__file__).with_name("libddtree.so")

DDTREE_F32 = 0
DDTREE_BF16 = 1
STATUS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP"}

_lib = None


class DDTreeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libddtree.so (built in-tree by ``python -m tree_verify_mla_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is not built; run `python -m tree_verify_mla_amd.build`")
    lib = ctypes.CDLL(str(LIB_PATH))
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.ddtree_abi_version.restype = I
    lib.ddtree_abi_version.argtypes = []
    lib.ddtree_last_error.restype = ctypes.c_char_p
    lib.ddtree_last_error.argtypes = []
    lib.ddtree_build_tree.restype = I
    lib.ddtree_build_tree.argtypes = [P, P, P, P, I, I, I, I, P, P, P, P, P]
    lib.ddtree_build_tree_visibility.restype = I
    lib.ddtree_build_tree_visibility.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P,
                                                 P]
    lib.ddtree_compile_visibility.restype = I
    lib.ddtree_compile_visibility.argtypes = [P, P, P, P, I, I, I, P, P, P, P, P]
    lib.ddtree_verify_attn_workspace_size.restype = SZ
    lib.ddtree_verify_attn_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.ddtree_verify_attn_plan.restype = I
    lib.ddtree_verify_attn_plan.argtypes = [I, I, I, I, I, I, P, P]
    lib.ddtree_verify_attn.restype = I
    lib.ddtree_verify_attn.argtypes = [P, P, I64, P, P, P, P, I, I, I, I, I, F, I, P, P, I, P, SZ, P]
    lib.ddtree_verify_attn_layers_workspace_size.restype = SZ
    lib.ddtree_verify_attn_layers_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.ddtree_verify_attn_layers.restype = I
    lib.ddtree_verify_attn_layers.argtypes = [I, P, I64, P, I64, I64, P, P, P, P, I, I, I, I, I, F,
                                              I, P, I64, P, I64, I, P, SZ, P]
    lib.ddtree_accept.restype = I
    lib.ddtree_accept.argtypes = [P, P, P, P, I, I, P, P, P, P, P]
    lib.ddtree_drafter_topk_workspace_size.restype = SZ
    lib.ddtree_drafter_topk_workspace_size.argtypes = [I, I, I]
    lib.ddtree_drafter_topk.restype = I
    lib.ddtree_drafter_topk.argtypes = [P, I, I, I, I, P, P, P, SZ, P]
    lib.ddtree_tree_sample.restype = I
    lib.ddtree_tree_sample_workspace_size.restype = SZ
    lib.ddtree_tree_sample_workspace_size.argtypes = [I]
    lib.ddtree_tree_sample.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P, P, P, P, SZ, P]
    lib.ddtree_commit_kv.restype = I
    lib.ddtree_commit_kv.argtypes = [P, P, P, P, P, I, I, I, P, P, ctypes.c_longlong, P,
                                     ctypes.c_longlong, I, P]
    lib.ddtree_tree_sample_noalloc.restype = I
    lib.ddtree_tree_sample_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P, P, P, P]
    lib.ddtree_validate_inputs.restype = I
    lib.ddtree_validate_inputs.argtypes = [I, P, I, P, P, I64, I64, P, P, P, P]
    lib.ddtree_probe_mfma_loop.restype = I
    lib.ddtree_probe_mfma_loop.argtypes = [I, I, P, P]
    lib.ddtree_device_info.restype = I
    lib.ddtree_device_info.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    _lib = lib
    return lib


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise DDTreeError(fn, rc, load().ddtree_last_error().decode(errors="replace"))


def _p(t: Optional[torch.Tensor], dtype=None, name: str = "tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def ddtree_abi_version() -> int:
    return load().ddtree_abi_version()


def ddtree_build_tree(topk_logprobs, topk_ids, root_tokens, qo_indptr, max_budget: int,
                      node_tokens, node_parents, node_depths, node_scores=None, stream=None):
    bs, D, K = topk_logprobs.shape
    _check("ddtree_build_tree", load().ddtree_build_tree(
        _p(topk_logprobs, torch.float32, "topk_logprobs"), _p(topk_ids, torch.int32, "topk_ids"),
        _p(root_tokens, torch.int32, "root_tokens"), _p(qo_indptr, torch.int32, "qo_indptr"),
        bs, D, K, int(max_budget), _p(node_tokens, torch.int32, "node_tokens"),
        _p(node_parents, torch.int32, "node_parents"), _p(node_depths, torch.int32, "node_depths"),
        _p(node_scores, torch.float32, "node_scores"), _stream(stream)))


def ddtree_build_tree_visibility(topk_logprobs, topk_ids, root_tokens, qo_indptr, prefix_lens,
                                 max_budget: int, max_q_len: int, node_tokens, node_parents,
                                 node_depths, vis_bits, node_scores=None, positions=None,
                                 stream=None):
    bs, D, K = topk_logprobs.shape
    _check("ddtree_build_tree_visibility", load().ddtree_build_tree_visibility(
        _p(topk_logprobs, torch.float32, "topk_logprobs"), _p(topk_ids, torch.int32, "topk_ids"),
        _p(root_tokens, torch.int32, "root_tokens"), _p(qo_indptr, torch.int32, "qo_indptr"),
        _p(prefix_lens, torch.int32, "prefix_lens"), bs, D, K, int(max_budget), int(max_q_len),
        vis_bits.shape[1], _p(node_tokens, torch.int32, "node_tokens"),
        _p(node_parents, torch.int32, "node_parents"), _p(node_depths, torch.int32, "node_depths"),
        _p(node_scores, torch.float32, "node_scores"), _p(vis_bits, torch.int32, "vis_bits"),
        _p(positions, torch.int64, "positions"), _stream(stream)))


def ddtree_compile_visibility(node_parents, node_depths, qo_indptr, prefix_lens, max_q_len: int,
                              vis_bits, positions=None, dense_mask=None, mask_indptr=None,
                              stream=None):
    bs = qo_indptr.numel() - 1
    W = vis_bits.shape[1]
    _check("ddtree_compile_visibility", load().ddtree_compile_visibility(
        _p(node_parents, torch.int32, "node_parents"), _p(node_depths, torch.int32, "node_depths"),
        _p(qo_indptr, torch.int32, "qo_indptr"), _p(prefix_lens, torch.int32, "prefix_lens"),
        bs, int(max_q_len), W, _p(vis_bits, torch.int32, "vis_bits"),
        _p(positions, torch.int64, "positions"), _p(dense_mask, torch.uint8, "dense_mask"),
        _p(mask_indptr, torch.int64, "mask_indptr"), _stream(stream)))


def ddtree_verify_attn_plan(bs: int, num_heads: int, max_q_len: int, max_kv_len: int,
                            num_splits: int, dtype: int) -> tuple:
    """(tile_rows, splits) of the verify-attention kernel these bounds select."""
    rows, splits = ctypes.c_int(0), ctypes.c_int(0)
    _check("ddtree_verify_attn_plan",
           load().ddtree_verify_attn_plan(bs, num_heads, max_q_len, max_kv_len, num_splits, dtype,
                                          ctypes.byref(rows), ctypes.byref(splits)))
    return rows.value, splits.value


def ddtree_verify_attn_workspace_size(bs: int, num_heads: int, max_q_len: int, max_kv_len: int,
                                      num_splits: int, dtype: int) -> int:
    return int(load().ddtree_verify_attn_workspace_size(bs, num_heads, max_q_len, max_kv_len,
                                                        num_splits, dtype))


def ddtree_verify_attn(q, kv_pool, kv_indptr, kv_indices, qo_indptr, vis_bits, max_q_len: int,
                       max_kv_len: int, scale: float, out, lse=None, num_splits: int = 0,
                       workspace=None, stream=None):
    if q.dtype == torch.bfloat16:
        dt = DDTREE_BF16
    elif q.dtype == torch.float32:
        dt = DDTREE_F32
    else:
        raise TypeError("q must be bfloat16 or float32")
    total_q, H, width = q.shape
    bs = qo_indptr.numel() - 1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ddtree_verify_attn", load().ddtree_verify_attn(
        _p(q, q.dtype, "q"), _p(kv_pool, q.dtype, "kv_pool"), int(kv_pool.shape[0]),
        _p(kv_indptr, torch.int32, "kv_indptr"), _p(kv_indices, torch.int32, "kv_indices"),
        _p(qo_indptr, torch.int32, "qo_indptr"), _p(vis_bits, torch.int32, "vis_bits"),
        vis_bits.shape[1], bs, H, int(max_q_len), int(max_kv_len), float(scale), dt,
        _p(out, q.dtype, "out"), _p(lse, torch.float32, "lse"), int(num_splits),
        _p(workspace, None, "workspace"), ws_bytes, _stream(stream)))


def ddtree_verify_attn_layers_workspace_size(num_layers: int, bs: int, num_heads: int,
                                             max_q_len: int, max_kv_len: int, num_splits: int,
                                             dtype: int) -> int:
    return int(load().ddtree_verify_attn_layers_workspace_size(
        num_layers, bs, num_heads, max_q_len, max_kv_len, num_splits, dtype))


def ddtree_verify_attn_layers(q, kv_pool, kv_indptr, kv_indices, qo_indptr, vis_bits,
                              max_q_len: int, max_kv_len: int, scale: float, out, lse=None,
                              num_splits: int = 0, workspace=None, stream=None):
    """q [L, total_q, H, 576], kv_pool [L, num_slots, 576] (or [1, ...]: one
    pool for every layer), out [L, total_q, H, 512], lse None or [L, total_q, H]."""
    if q.dtype == torch.bfloat16:
        dt = DDTREE_BF16
    elif q.dtype == torch.float32:
        dt = DDTREE_F32
    else:
        raise TypeError("q must be bfloat16 or float32")
    L, total_q, H, width = q.shape
    if kv_pool.dim() != 3 or kv_pool.shape[0] not in (1, L):
        raise ValueError("kv_pool must be [L, num_slots, 576] or [1, num_slots, 576]")
    if out.shape[0] != L or (lse is not None and lse.shape[0] != L):
        raise ValueError("out and lse need one entry per layer")
    if L > 1 and (out.stride(0) < out[0].numel() or
                  (lse is not None and lse.stride(0) < lse[0].numel())):
        raise ValueError("layer outputs must not overlap")
    bs = qo_indptr.numel() - 1
    kv_ls = kv_pool.stride(0) if kv_pool.shape[0] == L and L > 1 else 0
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ddtree_verify_attn_layers", load().ddtree_verify_attn_layers(
        L, _p(q, q.dtype, "q"), q.stride(0), _p(kv_pool, q.dtype, "kv_pool"), kv_ls,
        int(kv_pool.shape[1]),
        _p(kv_indptr, torch.int32, "kv_indptr"), _p(kv_indices, torch.int32, "kv_indices"),
        _p(qo_indptr, torch.int32, "qo_indptr"), _p(vis_bits, torch.int32, "vis_bits"),
        vis_bits.shape[1], bs, H, int(max_q_len), int(max_kv_len), float(scale), dt,
        _p(out, q.dtype, "out"), out.stride(0), _p(lse, torch.float32, "lse"),
        0 if lse is None else lse.stride(0), int(num_splits),
        _p(workspace, None, "workspace"), ws_bytes, _stream(stream)))


def ddtree_accept(node_tokens, node_parents, qo_indptr, target_predict, depth_max: int,
                  accepted_nodes, accept_len, commit_tokens, bonus_tokens, stream=None):
    bs = qo_indptr.numel() - 1
    _check("ddtree_accept", load().ddtree_accept(
        _p(node_tokens, torch.int32, "node_tokens"), _p(node_parents, torch.int32, "node_parents"),
        _p(qo_indptr, torch.int32, "qo_indptr"), _p(target_predict, torch.int32, "target_predict"),
        bs, int(depth_max), _p(accepted_nodes, torch.int32, "accepted_nodes"),
        _p(accept_len, torch.int32, "accept_len"), _p(commit_tokens, torch.int32, "commit_tokens"),
        _p(bonus_tokens, torch.int32, "bonus_tokens"), _stream(stream)))


def ddtree_commit_kv(kv_indptr, kv_indices, qo_indptr, accepted_nodes, accept_len,
                     max_kv_len: int, new_kv_indptr, new_kv_indices, kv_pool=None, stream=None):
    """Index form without ``kv_pool``; move form (rows compacted in place) with it."""
    bs = qo_indptr.numel() - 1
    depth_max = accepted_nodes.shape[1] - 1
    pool_ptr, nslots, dt = None, 0, DDTREE_BF16
    if kv_pool is not None:
        if kv_pool.dtype == torch.bfloat16:
            dt = DDTREE_BF16
        elif kv_pool.dtype == torch.float32:
            dt = DDTREE_F32
        else:
            raise TypeError("kv_pool must be bfloat16 or float32")
        if kv_pool.dim() != 2 or kv_pool.shape[1] != 576:
            raise ValueError("kv_pool must be [num_slots, 576]")
        pool_ptr, nslots = _p(kv_pool, kv_pool.dtype, "kv_pool"), int(kv_pool.shape[0])
    _check("ddtree_commit_kv", load().ddtree_commit_kv(
        _p(kv_indptr, torch.int32, "kv_indptr"), _p(kv_indices, torch.int32, "kv_indices"),
        _p(qo_indptr, torch.int32, "qo_indptr"), _p(accepted_nodes, torch.int32, "accepted_nodes"),
        _p(accept_len, torch.int32, "accept_len"), bs, int(depth_max), int(max_kv_len),
        _p(new_kv_indptr, torch.int32, "new_kv_indptr"),
        _p(new_kv_indices, torch.int32, "new_kv_indices"), int(new_kv_indices.numel()),
        pool_ptr, nslots, dt, _stream(stream)))


def ddtree_drafter_topk_workspace_size(rows: int, vocab: int, topk: int) -> int:
    return int(load().ddtree_drafter_topk_workspace_size(rows, vocab, topk))


def ddtree_drafter_topk(logits, topk_logprobs, topk_ids, workspace=None, stream=None):
    """logits [rows, vocab] (f32 or bf16) -> topk_logprobs [rows, k] f32, topk_ids [rows, k] i32."""
    if logits.dtype == torch.bfloat16:
        dt = DDTREE_BF16
    elif logits.dtype == torch.float32:
        dt = DDTREE_F32
    else:
        raise TypeError("logits must be bfloat16 or float32")
    rows, vocab = logits.shape
    k = topk_ids.shape[-1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ddtree_drafter_topk", load().ddtree_drafter_topk(
        _p(logits, logits.dtype, "logits"), dt, rows, vocab, k,
        _p(topk_logprobs, torch.float32, "topk_logprobs"), _p(topk_ids, torch.int32, "topk_ids"),
        _p(workspace, None, "workspace"), ws_bytes, _stream(stream)))


def ddtree_tree_sample_workspace_size(total_q: int) -> int:
    return int(load().ddtree_tree_sample_workspace_size(total_q))


def ddtree_tree_sample(node_tokens, node_parents, qo_indptr, target_probs, coins, bonus_uniforms,
                       depth_max: int, accepted_nodes, accept_len, commit_tokens, bonus_tokens,
                       workspace=None, stream=None):
    """Stochastic acceptance; target_probs [total_q, vocab] f32.  ``workspace``
    is caller-owned (ddtree_tree_sample_workspace_size(total_q) bytes), as for
    every other call: nothing is allocated here, so the call can be captured
    in a graph."""
    bs = qo_indptr.numel() - 1
    total_q, vocab = target_probs.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ddtree_tree_sample", load().ddtree_tree_sample(
        _p(node_tokens, torch.int32, "node_tokens"), _p(node_parents, torch.int32, "node_parents"),
        _p(qo_indptr, torch.int32, "qo_indptr"), _p(target_probs, torch.float32, "target_probs"),
        _p(coins, torch.float32, "coins"), _p(bonus_uniforms, torch.float32, "bonus_uniforms"),
        bs, int(total_q), int(depth_max), int(vocab),
        _p(accepted_nodes, torch.int32, "accepted_nodes"),
        _p(accept_len, torch.int32, "accept_len"), _p(commit_tokens, torch.int32, "commit_tokens"),
        _p(bonus_tokens, torch.int32, "bonus_tokens"), _p(workspace, None, "workspace"), ws_bytes,
        _stream(stream)))


DDTREE_NUM_CHECKS = 5
CHECK_NAMES = ("QO_INDPTR", "KV_INDPTR", "KV_LEN", "KV_INDEX", "PARENT")


def ddtree_validate_inputs(qo_indptr, total_q: int, kv_indptr, kv_indices, num_slots: int,
                           report, prefix_lens=None, node_parents=None, stream=None):
    """Debug check of a step's index arrays; ``report`` is an int32 device
    tensor of 2 * DDTREE_NUM_CHECKS entries (count, first offending index)."""
    bs = qo_indptr.numel() - 1
    if report.numel() < 2 * DDTREE_NUM_CHECKS:
        raise ValueError("report needs 2 * DDTREE_NUM_CHECKS entries")
    _check("ddtree_validate_inputs", load().ddtree_validate_inputs(
        bs, _p(qo_indptr, torch.int32, "qo_indptr"), int(total_q),
        _p(kv_indptr, torch.int32, "kv_indptr"), _p(kv_indices, torch.int32, "kv_indices"),
        int(kv_indices.numel()), int(num_slots), _p(prefix_lens, torch.int32, "prefix_lens"),
        _p(node_parents, torch.int32, "node_parents"), _p(report, torch.int32, "report"),
        _stream(stream)))


def ddtree_tree_sample_noalloc(node_tokens, node_parents, qo_indptr, target_probs, coins,
                               bonus_uniforms, depth_max: int, accepted_nodes, accept_len,
                               commit_tokens, bonus_tokens, stream=None):
    """ddtree_tree_sample on the library's built-in scratch (no workspace,
    at most 4096 tree nodes)."""
    bs = qo_indptr.numel() - 1
    total_q, vocab = target_probs.shape
    _check("ddtree_tree_sample_noalloc", load().ddtree_tree_sample_noalloc(
        _p(node_tokens, torch.int32, "node_tokens"), _p(node_parents, torch.int32, "node_parents"),
        _p(qo_indptr, torch.int32, "qo_indptr"), _p(target_probs, torch.float32, "target_probs"),
        _p(coins, torch.float32, "coins"), _p(bonus_uniforms, torch.float32, "bonus_uniforms"),
        bs, int(total_q), int(depth_max), int(vocab),
        _p(accepted_nodes, torch.int32, "accepted_nodes"),
        _p(accept_len, torch.int32, "accept_len"), _p(commit_tokens, torch.int32, "commit_tokens"),
        _p(bonus_tokens, torch.int32, "bonus_tokens"), _stream(stream)))


def ddtree_probe_mfma_loop(grid: int, iters: int, out, stream=None) -> int:
    """Launch the matrix-core loop probe; returns its flops per launch."""
    if out.numel() < grid * 256:
        raise ValueError("out must hold grid * 256 floats")
    _check("ddtree_probe_mfma_loop", load().ddtree_probe_mfma_loop(
        int(grid), int(iters), _p(out, torch.float32, "out"), _stream(stream)))
    return grid * 4 * iters * 8 * 32768


def ddtree_device_info():
    """(compute units, peak shader clock in kHz) of the current device."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    _check("ddtree_device_info", load().ddtree_device_info(ctypes.byref(cus), ctypes.byref(khz)))
    return cus.value, khz.value
