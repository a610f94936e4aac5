"""Python binding of libtreeverify (tree-based speculative verification on
MI355X).

Thin ctypes wrappers with the names of the C entry points in
include/treeverify.h.  They only marshal arguments: sizes come from tensor
shapes, pointers from Tensor.data_ptr(), the stream from torch's current
stream.  All work happens in the HIP library; a non-OK return raises
TreeVerifyError.  PyTorch is used for device memory and streams only.
"""
import ctypes
import os

__all__ = [
    "TreeVerifyError", "lib", "lib_path", "TV_F32", "TV_BF16", "EXPORTS",
    "tree_build_mask", "tree_attn_verify_workspace", "tree_attn_verify",
    "tree_verify_workspace", "tree_verify_greedy", "tree_verify_mss", "kv_commit_accepted",
    "tree_verify_naive", "tree_logits_transform", "TV_OUT_LOGITS", "TV_OUT_PROBS", "tv_status_string",
    "tree_verify_mss_commit", "tree_verify_mss_multi", "tree_mask_attn_verify", "tree_verify_mss_noalloc",
    "TV_NOALLOC_SCRATCH_BYTES",
]

TV_F32 = 0
TV_BF16 = 1
TV_OUT_LOGITS = 0
TV_OUT_PROBS = 1
EXPORTS = ("tree_build_mask", "tree_attn_verify_workspace", "tree_attn_verify",
           "tree_verify_workspace", "tree_verify_greedy", "tree_verify_mss",
           "kv_commit_accepted", "tree_verify_naive", "tree_logits_transform", "tv_status_string",
           "tree_verify_mss_commit", "tree_verify_mss_multi", "tree_mask_attn_verify",
           "tree_verify_mss_noalloc")
TV_NOALLOC_SCRATCH_BYTES = 4 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libtreeverify.so")


class TreeVerifyError(RuntimeError):
    pass


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with "
                          "`python -m tree_speculative_verification_attn_amd.build`")
    L = ctypes.CDLL(lib_path)
    P, I, U64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "tree_build_mask": ([I, I, P, P, P, P, P, P], I),
        "tree_attn_verify_workspace": ([I, I, I, I, I, I], SZ),
        "tree_attn_verify": ([I, I, I, I, I, F, P, P, P, I, I, P, I, P, P, P, P, P, SZ, P], I),
        "tree_mask_attn_verify": ([I, I, I, I, I, F, P, P, P, I, I, P, I, P, P, P, P, P, P, P, P, SZ, P], I),
        "tree_verify_workspace": ([I, I, I], SZ),
        "tree_verify_greedy": ([I, I, I, P, P, P, P, P, P, P, P, SZ, P], I),
        "tree_verify_mss": ([I, I, I, I, P, P, P, P, P, P, U64, U64, P, P, P, P, P, SZ, P], I),
        "tree_verify_mss_noalloc": ([I, I, I, I, P, P, P, P, P, P, U64, U64, P, P, P, P, P], I),
        "kv_commit_accepted": ([I, I, I, I, I, P, P, I, I, P, I, P, P, P, P, P], I),
        "tree_verify_mss_commit": ([I, I, I, I, P, P, P, P, P, P, U64, U64, P, P, P, P, P, SZ,
                                    I, I, I, P, P, I, I, P, I, P, P], I),
        "tree_verify_mss_multi": ([I, I, I, I, I, P, P, P, P, P, P, P, U64, U64, P, P, P, P, P, SZ, P], I),
        "tree_logits_transform": ([I, I, P, P, F, I, F, I, P], I),
        "tree_verify_naive": ([I, I, I, P, P, P, P, U64, U64, P, P, P, P, SZ, P], I),
        "tv_status_string": ([I], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


_LIB = None


def lib():
    """The loaded library (loaded on first use; ImportError if it is missing)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def tv_status_string(code: int) -> str:
    return lib().tv_status_string(int(code)).decode()


def _check(code, what):
    if code != 0:
        raise TreeVerifyError(f"{what}: {tv_status_string(code)} ({code})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return TV_F32
    if t.dtype == torch.bfloat16:
        return TV_BF16
    raise TreeVerifyError(f"unsupported dtype {t.dtype}")


def tree_build_mask(parent, anc, child, depth, status, stream=None):
    """parent [B][N] int32 -> anc [B][N] u64 (int64 tensor), child [B][N+1],
    depth [B][N] int32, status [B] int32."""
    B, N = parent.shape
    _check(lib().tree_build_mask(B, N, _ptr(parent), _ptr(anc), _ptr(child), _ptr(depth),
                               _ptr(status), _stream(stream)), "tree_build_mask")


def tree_attn_verify_workspace(dtype_code, B, N, H, D, max_blocks):
    return int(lib().tree_attn_verify_workspace(dtype_code, B, N, H, D, max_blocks))


def tree_attn_verify(q, k_cache, v_cache, block_table, prefix_len, anc, status, out, workspace,
                     scale=None, stream=None):
    """q [B][N][H][D], k/v_cache [num_blocks][H][16][D], block_table [B][max_blocks]."""
    B, N, H, D = q.shape
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().tree_attn_verify(_dtype_code(q), B, N, H, D, float(scale), _ptr(q), _ptr(k_cache),
                                _ptr(v_cache), k_cache.shape[0], k_cache.shape[2], _ptr(block_table),
                                block_table.shape[1], _ptr(prefix_len), _ptr(anc), _ptr(status),
                                _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
           "tree_attn_verify")


def tree_mask_attn_verify(q, k_cache, v_cache, block_table, prefix_len, parent, anc, child, depth,
                          status, out, workspace, scale=None, stream=None):
    """tree_build_mask then tree_attn_verify, one launch where the plan allows."""
    B, N, H, D = q.shape
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().tree_mask_attn_verify(_dtype_code(q), B, N, H, D, float(scale), _ptr(q), _ptr(k_cache),
                                     _ptr(v_cache), k_cache.shape[0], k_cache.shape[2], _ptr(block_table),
                                     block_table.shape[1], _ptr(prefix_len), _ptr(parent), _ptr(anc),
                                     _ptr(child), _ptr(depth), _ptr(status), _ptr(out), _ptr(workspace),
                                     ws_bytes, _stream(stream)), "tree_mask_attn_verify")


def tree_verify_workspace(B, N, V):
    return int(lib().tree_verify_workspace(B, N, V))


def tree_verify_greedy(target_logits, token, child, status, accepted, num_accepted, bonus,
                       workspace, stream=None):
    B, N1, V = target_logits.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tree_verify_greedy(B, N1 - 1, V, _ptr(target_logits), _ptr(token), _ptr(child),
                                  _ptr(status), _ptr(accepted), _ptr(num_accepted), _ptr(bonus),
                                  _ptr(workspace), ws_bytes, _stream(stream)), "tree_verify_greedy")


def tree_verify_mss(target_logits, ssm_probs, q_row, token, child, status, seed, offset,
                    accepted, num_accepted, bonus, rounds, workspace, stream=None):
    B, N1, V = target_logits.shape
    R = ssm_probs.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tree_verify_mss(B, N1 - 1, V, R, _ptr(target_logits), _ptr(ssm_probs), _ptr(q_row),
                               _ptr(token), _ptr(child), _ptr(status), int(seed), int(offset),
                               _ptr(accepted), _ptr(num_accepted), _ptr(bonus), _ptr(rounds),
                               _ptr(workspace), ws_bytes, _stream(stream)), "tree_verify_mss")


def tree_verify_mss_noalloc(target_logits, ssm_probs, q_row, token, child, status, seed, offset,
                            accepted, num_accepted, bonus, rounds, stream=None):
    """tree_verify_mss with the library's fixed device scratch as its
    workspace: allocates nothing."""
    B, N1, V = target_logits.shape
    R = ssm_probs.shape[1]
    _check(lib().tree_verify_mss_noalloc(B, N1 - 1, V, R, _ptr(target_logits), _ptr(ssm_probs), _ptr(q_row),
                                       _ptr(token), _ptr(child), _ptr(status), int(seed), int(offset),
                                       _ptr(accepted), _ptr(num_accepted), _ptr(bonus), _ptr(rounds),
                                       _stream(stream)), "tree_verify_mss_noalloc")


def tree_verify_mss_commit(target_logits, ssm_probs, q_row, token, child, status, seed, offset,
                           accepted, num_accepted, bonus, rounds, workspace,
                           k_cache, v_cache, block_table, prefix_len, stream=None):
    """tree_verify_mss followed by kv_commit_accepted of its path, in one launch."""
    B, N1, V = target_logits.shape
    R = ssm_probs.shape[1]
    nb, H, bs, D = k_cache.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tree_verify_mss_commit(B, N1 - 1, V, R, _ptr(target_logits), _ptr(ssm_probs), _ptr(q_row),
                                      _ptr(token), _ptr(child), _ptr(status), int(seed), int(offset),
                                      _ptr(accepted), _ptr(num_accepted), _ptr(bonus), _ptr(rounds),
                                      _ptr(workspace), ws_bytes, _dtype_code(k_cache), H, D, _ptr(k_cache),
                                      _ptr(v_cache), nb, bs, _ptr(block_table), block_table.shape[1],
                                      _ptr(prefix_len), _stream(stream)), "tree_verify_mss_commit")


def tree_verify_mss_multi(target_logits, ssm_probs, prop_node, prop_row, token, child, status, seed, offset,
                          accepted, num_accepted, bonus, rounds, workspace, stream=None):
    """MSS over proposals: prop_node / prop_row [B][S] int32 (node -1 = unused slot)."""
    B, N1, V = target_logits.shape
    R = ssm_probs.shape[1]
    S = prop_node.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tree_verify_mss_multi(B, N1 - 1, S, V, R, _ptr(target_logits), _ptr(ssm_probs), _ptr(prop_node),
                                     _ptr(prop_row), _ptr(token), _ptr(child), _ptr(status), int(seed), int(offset),
                                     _ptr(accepted), _ptr(num_accepted), _ptr(bonus), _ptr(rounds),
                                     _ptr(workspace), ws_bytes, _stream(stream)), "tree_verify_mss_multi")


def tree_verify_naive(target_logits, token, child, status, seed, offset, accepted, num_accepted, bonus,
                      workspace, stream=None):
    B, N1, V = target_logits.shape
    N = N1 - 1
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tree_verify_naive(B, N, V, _ptr(target_logits), _ptr(token), _ptr(child), _ptr(status),
                                   int(seed), int(offset), _ptr(accepted), _ptr(num_accepted), _ptr(bonus),
                                   _ptr(workspace), ws_bytes, _stream(stream)), "tree_verify_naive")


def kv_commit_accepted(k_cache, v_cache, block_table, prefix_len, accepted, num_accepted, status,
                       stream=None):
    nb, H, bs, D = k_cache.shape
    B, N = accepted.shape
    _check(lib().kv_commit_accepted(_dtype_code(k_cache), B, N, H, D, _ptr(k_cache), _ptr(v_cache), nb,
                                  bs, _ptr(block_table), block_table.shape[1], _ptr(prefix_len),
                                  _ptr(accepted), _ptr(num_accepted), _ptr(status), _stream(stream)),
           "kv_commit_accepted")


def tree_logits_transform(logits, out, temperature=1.0, top_k=0, top_p=1.0, kind=TV_OUT_LOGITS,
                          stream=None):
    """logits / out: fp32 [..., V] (out may be logits itself); every row is transformed."""
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    _check(lib().tree_logits_transform(rows, V, _ptr(logits), _ptr(out), float(temperature), int(top_k),
                                       float(top_p), int(kind), _stream(stream)),
           "tree_logits_transform")
