"""ctypes binding of libddt.so (C ABI in include/ddt.h).

Argument marshalling only: every step of the verify path runs in the library's HIP
kernels.  PyTorch provides device memory (outputs and workspaces are torch tensors)
and the current stream.  There is no fallback: if the library is missing or the
tensors are not on a GPU, the calls raise.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libddt.so")

DDT_OK, DDT_ERR_ARG, DDT_ERR_UNSUPPORTED, DDT_ERR_WORKSPACE, DDT_ERR_HIP = range(5)
DDT_F32, DDT_BF16 = 0, 1

EXPORTS = ("ddt_status_string", "ddt_last_error", "ddt_abi_version",
           "ddt_build_tree_workspace", "ddt_build_tree",
           "ddt_build_tree_noalloc_max_scratch", "ddt_build_tree_noalloc",
           "ddt_tree_attn_workspace", "ddt_tree_attn",
           "ddt_tree_attn_rope_workspace", "ddt_tree_attn_rope", "ddt_tree_rope",
           "ddt_tree_attn_paged_workspace", "ddt_tree_attn_paged", "ddt_commit_paged",
           "ddt_tree_accept_sampled",
           "ddt_gdn_tree_step_workspace", "ddt_gdn_tree_step", "ddt_gdn_tree_step_deferred", "ddt_gdn_tree_states",
           "ddt_tree_accept_workspace", "ddt_tree_accept",
           "ddt_commit", "ddt_gdn_replay")


class DDTError(RuntimeError):
    """A libddt call returned a non-zero status."""

    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (%s)" % (fn, _status_name(status), msg))
        self.status = status


class KVLayer(ctypes.Structure):
    _fields_ = [("k_tree", ctypes.c_void_p), ("v_tree", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p)]


class GDNLayer(ctypes.Structure):
    _fields_ = [("S_scratch", ctypes.c_void_p), ("S", ctypes.c_void_p),
                ("conv_scratch", ctypes.c_void_p), ("conv_state", ctypes.c_void_p)]


class GDNReplayLayer(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("conv_w", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("g", ctypes.c_void_p), ("S", ctypes.c_void_p),
                ("conv_state", ctypes.c_void_p)]


_lib = None
P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float


def lib():
    """Load libddt.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libddt.so is not built (%s); run "
                           "`python -m tree_speculative_decoding_ddt_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "ddt_status_string": (ctypes.c_char_p, [I]),
        "ddt_last_error": (ctypes.c_char_p, []),
        "ddt_abi_version": (I, []),
        "ddt_build_tree_workspace": (Z, [I, I, I, I, I]),
        "ddt_build_tree": (I, [P, I, I, I, I, I, I, P, P, P, P, P, P, P, Z, P]),
        "ddt_build_tree_noalloc_max_scratch": (Z, []),
        "ddt_build_tree_noalloc": (I, [P, I, I, I, I, I, I, P, P, P, P, P, P, P]),
        "ddt_tree_attn_workspace": (Z, [I, I, I, I, I, I, I]),
        "ddt_tree_attn": (I, [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, Z, P]),
        "ddt_tree_attn_rope_workspace": (Z, [I, I, I, I, I, I, I]),
        "ddt_tree_attn_paged_workspace": (Z, [I, I, I, I, I, I, I, I]),
        "ddt_tree_accept_sampled": (I, [P, I, P, P, P, P, I, I, I, I, P, P, P, P, Z, P]),
        "ddt_tree_rope": (I, [P, P, P, P, P, I, F, I, I, I, I, I, I, P, P, P, P]),
        "ddt_tree_attn_paged": (I, [P, P, P, P, I, I, I, P, P, P, P, I, I, I, I, I, F, I, P, P, Z, P]),
        "ddt_commit_paged": (I, [P, P, P, ctypes.POINTER(KVLayer), I, I, I, P, I, I, I, I,
                                 ctypes.POINTER(GDNLayer), I, I, I, I, I, I, I, I, I, I, P]),
        "ddt_tree_attn_rope": (I, [P, P, P, P, I, F, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, Z, P]),
        "ddt_gdn_tree_step_workspace": (Z, [I, I, I, I]),
        "ddt_gdn_tree_step": (I, [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, Z, P]),
        "ddt_gdn_tree_step_deferred": (I, [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, Z, P]),
        "ddt_gdn_tree_states": (I, [P, P, I, I, I, I, I, P, Z, P]),
        "ddt_tree_accept_workspace": (Z, [I, I, I]),
        "ddt_tree_accept": (I, [P, I, P, P, I, I, I, I, P, P, P, P, Z, P]),
        "ddt_commit": (I, [P, P, P, ctypes.POINTER(KVLayer), I, I, I, I, I,
                           ctypes.POINTER(GDNLayer), I, I, I, I, I, I, I, I, I, I, P]),
        "ddt_gdn_replay": (I, [P, P, ctypes.POINTER(GDNReplayLayer), I, I, I, I, I, I, I, I, I, I, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _status_name(status):
    try:
        return lib().ddt_status_string(status).decode()
    except Exception:  # noqa: BLE001 -- only used to format an error
        return str(status)


def _check(fn, status):
    if status != DDT_OK:
        raise DDTError(fn, status, lib().ddt_last_error().decode())


def _dt(t):
    if t.dtype == torch.float32:
        return DDT_F32
    if t.dtype == torch.bfloat16:
        return DDT_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libddt works on GPU tensors only")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ws(nbytes, dev, ws):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small: %d < %d bytes" % (ws.numel() * ws.element_size(), nbytes))
        return ws
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)


# ---------------------------------------------------------------- workspace queries

def build_tree_workspace(n, L, V, B, K=0):
    return lib().ddt_build_tree_workspace(n, L, V, B, K)


def tree_attn_workspace(n, B, Hq, Hkv, D, Pmax, dtype):
    return lib().ddt_tree_attn_workspace(n, B, Hq, Hkv, D, Pmax, DDT_BF16 if dtype == torch.bfloat16 else DDT_F32)


def tree_attn_rope_workspace(n, B, Hq, Hkv, D, Pmax, dtype):
    return lib().ddt_tree_attn_rope_workspace(n, B, Hq, Hkv, D, Pmax, DDT_BF16 if dtype == torch.bfloat16 else DDT_F32)


def tree_attn_paged_workspace(n, B, Hq, Hkv, D, max_blocks, page_size, dtype):
    return lib().ddt_tree_attn_paged_workspace(n, B, Hq, Hkv, D, max_blocks, page_size,
                                               DDT_BF16 if dtype == torch.bfloat16 else DDT_F32)


def gdn_tree_step_workspace(n, B, H, dk):
    return lib().ddt_gdn_tree_step_workspace(n, B, H, dk)


def tree_accept_workspace(n, B, V):
    return lib().ddt_tree_accept_workspace(n, B, V)


# ---------------------------------------------------------------- calls

def build_tree(draft_logits, B, root_token, K=0, ws=None, out=None):
    """draft_logits [n][L][V] (f32/bf16), root_token [n] int32 ->
    dict tok, parent, depth [n][B+1] int32, score [n][B+1] f32, anc [n][B+1] int64 (u64 bits)."""
    _gpu(draft_logits, root_token)
    n, L, V = draft_logits.shape
    dev = draft_logits.device
    T = B + 1
    if out is None:
        out = {"tok": torch.empty(n, T, dtype=torch.int32, device=dev),
               "parent": torch.empty(n, T, dtype=torch.int32, device=dev),
               "depth": torch.empty(n, T, dtype=torch.int32, device=dev),
               "score": torch.empty(n, T, dtype=torch.float32, device=dev),
               "anc": torch.empty(n, T, dtype=torch.int64, device=dev)}
    nb = lib().ddt_build_tree_workspace(n, L, V, B, K)
    w = _ws(nb, dev, ws)
    _check("ddt_build_tree", lib().ddt_build_tree(
        _ptr(draft_logits), _dt(draft_logits), n, L, V, B, K, _ptr(root_token), _ptr(out["tok"]),
        _ptr(out["parent"]), _ptr(out["depth"]), _ptr(out["score"]), _ptr(out["anc"]),
        _ptr(w), w.numel() * w.element_size(), _stream(dev)))
    return out


def build_tree_noalloc(draft_logits, B, root_token, K=0, out=None):
    """build_tree without a workspace: the library's static per-device scratch (for callers
    that cannot allocate; calls on one device must not overlap)."""
    _gpu(draft_logits, root_token)
    n, L, V = draft_logits.shape
    dev = draft_logits.device
    T = B + 1
    if out is None:
        out = {"tok": torch.empty(n, T, dtype=torch.int32, device=dev),
               "parent": torch.empty(n, T, dtype=torch.int32, device=dev),
               "depth": torch.empty(n, T, dtype=torch.int32, device=dev),
               "score": torch.empty(n, T, dtype=torch.float32, device=dev),
               "anc": torch.empty(n, T, dtype=torch.int64, device=dev)}
    _check("ddt_build_tree_noalloc", lib().ddt_build_tree_noalloc(
        _ptr(draft_logits), _dt(draft_logits), n, L, V, B, K, _ptr(root_token), _ptr(out["tok"]),
        _ptr(out["parent"]), _ptr(out["depth"]), _ptr(out["score"]), _ptr(out["anc"]), _stream(dev)))
    return out


def tree_attn(q, k_cache, v_cache, prefix_len, k_tree, v_tree, anc, scale=0.0, ws=None, out=None):
    """q [n][T][Hq][D], k/v_cache [n][Hkv][Pmax][D], prefix_len [n] int32, k/v_tree [n][Hkv][T][D],
    anc [n][T] int64 -> out [n][T][Hq][D] (dtype of q)."""
    _gpu(q, k_cache, v_cache, prefix_len, k_tree, v_tree, anc)
    n, T, Hq, D = q.shape
    Hkv, Pmax = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    dt = _dt(q)
    nb = lib().ddt_tree_attn_workspace(n, T - 1, Hq, Hkv, D, Pmax, dt)
    w = _ws(nb, dev, ws)
    _check("ddt_tree_attn", lib().ddt_tree_attn(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len), _ptr(k_tree), _ptr(v_tree), _ptr(anc),
        n, T - 1, Hq, Hkv, D, Pmax, float(scale), dt, _ptr(out), _ptr(w), w.numel() * w.element_size(),
        _stream(dev)))
    return out


def tree_attn_rope(q, k_new, v_new, depth, rot_dim, theta, k_cache, v_cache, prefix_len, anc, scale=0.0, ws=None,
                   out=None):
    """Pre-rotation q [n][T][Hq][D], k_new/v_new [n][T][Hkv][D], depth [n][T] int32 ->
    dict o [n][T][Hq][D], k_tree/v_tree [n][Hkv][T][D] (rotated keys / values, written)."""
    _gpu(q, k_new, v_new, depth, k_cache, v_cache, prefix_len, anc)
    n, T, Hq, D = q.shape
    Hkv, Pmax = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    if out is None:
        out = {"o": torch.empty_like(q), "k_tree": torch.empty(n, Hkv, T, D, dtype=q.dtype, device=dev),
               "v_tree": torch.empty(n, Hkv, T, D, dtype=q.dtype, device=dev)}
    dt = _dt(q)
    w = _ws(lib().ddt_tree_attn_rope_workspace(n, T - 1, Hq, Hkv, D, Pmax, dt), dev, ws)
    _check("ddt_tree_attn_rope", lib().ddt_tree_attn_rope(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(depth), int(rot_dim), float(theta), _ptr(k_cache), _ptr(v_cache),
        _ptr(prefix_len), _ptr(out["k_tree"]), _ptr(out["v_tree"]), _ptr(anc), n, T - 1, Hq, Hkv, D, Pmax,
        float(scale), dt, _ptr(out["o"]), _ptr(w), w.numel() * w.element_size(), _stream(dev)))
    return out


def tree_rope(q, k_new, v_new, depth, prefix_len, rot_dim, theta, out=None):
    """Rotation alone: -> dict q (rotated, [n][T][Hq][D]), k_tree/v_tree [n][Hkv][T][D]."""
    _gpu(q, k_new, v_new, depth, prefix_len)
    n, T, Hq, D = q.shape
    Hkv = k_new.shape[2]
    dev = q.device
    if out is None:
        out = {"q": torch.empty_like(q), "k_tree": torch.empty(n, Hkv, T, D, dtype=q.dtype, device=dev),
               "v_tree": torch.empty(n, Hkv, T, D, dtype=q.dtype, device=dev)}
    _check("ddt_tree_rope", lib().ddt_tree_rope(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(depth), _ptr(prefix_len), int(rot_dim), float(theta), n, T - 1, Hq,
        Hkv, D, _dt(q), _ptr(out["q"]), _ptr(out["k_tree"]), _ptr(out["v_tree"]), _stream(dev)))
    return out


def tree_attn_paged(q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, anc, scale=0.0, ws=None, out=None):
    """q [n][T][Hq][D], k/v_pages [num_pages][Hkv][page_size][D], block_table [n][max_blocks] int32,
    prefix_len [n] int32, k/v_tree [n][Hkv][T][D], anc [n][T] int64 -> out [n][T][Hq][D]."""
    _gpu(q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, anc)
    n, T, Hq, D = q.shape
    num_pages, Hkv, ps = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    maxb = block_table.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    dt = _dt(q)
    w = _ws(lib().ddt_tree_attn_paged_workspace(n, T - 1, Hq, Hkv, D, maxb, ps, dt), dev, ws)
    _check("ddt_tree_attn_paged", lib().ddt_tree_attn_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), maxb, ps, num_pages, _ptr(prefix_len),
        _ptr(k_tree), _ptr(v_tree), _ptr(anc), n, T - 1, Hq, Hkv, D, float(scale), dt, _ptr(out), _ptr(w),
        w.numel() * w.element_size(), _stream(dev)))
    return out


def gdn_tree_step(x, conv_w, conv_state, v, beta, g, S, parent, L, ws=None, out=None, store_states=True):
    """x [n][T][C], conv_w [C][W] f32, conv_state [n][W-1][C], v [n][T][H][dv], beta, g [n][T][H] f32,
    S [n][H][dv][dk] f32, parent [n][T] int32 -> dict o, S_scratch, conv_scratch.
    store_states=False stores no node state (scratch pointers NULL; the commit then uses gdn_replay)."""
    _gpu(x, conv_w, conv_state, v, beta, g, S, parent)
    n, T, C = x.shape
    W = conv_w.shape[1]
    H, dv, dk = S.shape[1], S.shape[2], S.shape[3]
    dev = x.device
    if out is None:
        out = {"o": torch.empty(n, T, H, dv, dtype=x.dtype, device=dev), "S_scratch": None, "conv_scratch": None}
        if store_states:
            out["S_scratch"] = torch.empty(n, T, H, dv, dk, dtype=torch.float32, device=dev)
            out["conv_scratch"] = torch.empty(n, T, W - 1, C, dtype=x.dtype, device=dev)
    # without state storage the scratch pointers are NULL (a caller's out keeps its buffers)
    Ssc = out["S_scratch"] if store_states else None
    csc = out["conv_scratch"] if store_states else None
    w = _ws(lib().ddt_gdn_tree_step_workspace(n, T - 1, H, dk), dev, ws)
    _check("ddt_gdn_tree_step", lib().ddt_gdn_tree_step(
        _ptr(x), _ptr(conv_w), _ptr(conv_state), _ptr(csc), _ptr(v), _ptr(beta), _ptr(g),
        _ptr(S), _ptr(Ssc), _ptr(out["o"]), _ptr(parent), n, T - 1, L, H, dk, dv, C, W,
        _dt(x), _ptr(w), w.numel() * w.element_size(), _stream(dev)))
    return out


def gdn_tree_step_deferred(x, conv_w, conv_state, v, beta, g, S, parent, L, ws, out=None):
    """The tree step without the node-state write (bf16): o and conv_scratch, with each node's
    k, w and path records left in ws (a uint8 tensor of gdn_tree_step_workspace bytes, which the
    caller keeps for gdn_tree_states) -> dict o, S_scratch (allocated, not written), conv_scratch."""
    _gpu(x, conv_w, conv_state, v, beta, g, S, parent, ws)
    n, T, C = x.shape
    W = conv_w.shape[1]
    H, dv, dk = S.shape[1], S.shape[2], S.shape[3]
    dev = x.device
    if out is None:
        out = {"o": torch.empty(n, T, H, dv, dtype=x.dtype, device=dev),
               "S_scratch": torch.empty(n, T, H, dv, dk, dtype=torch.float32, device=dev),
               "conv_scratch": torch.empty(n, T, W - 1, C, dtype=x.dtype, device=dev)}
    _check("ddt_gdn_tree_step_deferred", lib().ddt_gdn_tree_step_deferred(
        _ptr(x), _ptr(conv_w), _ptr(conv_state), _ptr(out["conv_scratch"]), _ptr(v), _ptr(beta), _ptr(g),
        _ptr(S), _ptr(out["o"]), _ptr(parent), n, T - 1, L, H, dk, dv, C, W,
        _dt(x), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return out


def gdn_tree_states(S, S_scratch, ws, stream=None):
    """Write every node's state into S_scratch [n][T][H][dv][dk] from S [n][H][dv][dk] and the ws a
    gdn_tree_step_deferred call left (on `stream`, a torch stream; default the current one)."""
    _gpu(S, S_scratch, ws)
    n, T, H, dv, dk = S_scratch.shape
    st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(S.device)
    _check("ddt_gdn_tree_states", lib().ddt_gdn_tree_states(
        _ptr(S), _ptr(S_scratch), n, T - 1, H, dk, dv, _ptr(ws), ws.numel() * ws.element_size(), st))
    return S_scratch


def tree_accept(target_logits, tok, parent, L, ws=None, out=None):
    """target_logits [n][T][V], tok/parent [n][T] int32 -> dict acc_rows [n][L+1], acc_len [n], bonus [n]."""
    _gpu(target_logits, tok, parent)
    n, T, V = target_logits.shape
    dev = target_logits.device
    if out is None:
        out = {"acc_rows": torch.empty(n, L + 1, dtype=torch.int32, device=dev),
               "acc_len": torch.empty(n, dtype=torch.int32, device=dev),
               "bonus": torch.empty(n, dtype=torch.int32, device=dev)}
    nb = lib().ddt_tree_accept_workspace(n, T - 1, V)
    w = _ws(nb, dev, ws)
    _check("ddt_tree_accept", lib().ddt_tree_accept(
        _ptr(target_logits), _dt(target_logits), _ptr(tok), _ptr(parent), n, T - 1, L, V,
        _ptr(out["acc_rows"]), _ptr(out["acc_len"]), _ptr(out["bonus"]), _ptr(w),
        w.numel() * w.element_size(), _stream(dev)))
    return out


def tree_accept_sampled(target_logits, gumbel, temperature, tok, parent, L, ws=None, out=None):
    """As tree_accept with each row's target token a Gumbel-max draw: gumbel [n][T][V] f32,
    temperature [n] f32 (<= 0: greedy)."""
    _gpu(target_logits, gumbel, temperature, tok, parent)
    n, T, V = target_logits.shape
    dev = target_logits.device
    if out is None:
        out = {"acc_rows": torch.empty(n, L + 1, dtype=torch.int32, device=dev),
               "acc_len": torch.empty(n, dtype=torch.int32, device=dev),
               "bonus": torch.empty(n, dtype=torch.int32, device=dev)}
    w = _ws(lib().ddt_tree_accept_workspace(n, T - 1, V), dev, ws)
    _check("ddt_tree_accept_sampled", lib().ddt_tree_accept_sampled(
        _ptr(target_logits), _dt(target_logits), _ptr(gumbel), _ptr(temperature), _ptr(tok), _ptr(parent), n, T - 1,
        L, V, _ptr(out["acc_rows"]), _ptr(out["acc_len"]), _ptr(out["bonus"]), _ptr(w), w.numel() * w.element_size(),
        _stream(dev)))
    return out


def commit(acc_rows, acc_len, prefix_len, kv_layers=(), gdn_layers=(), B=None, block_table=None, Pmax=None,
           page_size=None):
    """In-place commit.  kv_layers: sequence of (k_tree, v_tree, k_cache, v_cache);
    gdn_layers: sequence of (S_scratch, S, conv_scratch, conv_state).
    With block_table [n][max_blocks] int32, k_cache / v_cache are page pools
    [num_pages][Hkv][page_size][D] (ddt_commit_paged).
    The prefix capacity that guards overflow comes from the KV caches (Pmax rows, or
    max_blocks * page_size); with no KV layer it must be given (Pmax, or page_size with
    a block table)."""
    _gpu(acc_rows, acc_len, prefix_len)
    n, Lp1 = acc_rows.shape
    dev = acc_rows.device
    kv = (KVLayer * max(1, len(kv_layers)))()
    Hkv = D = 1
    kv_dt = DDT_BF16
    T = None
    for i, (kt, vt, kc, vc) in enumerate(kv_layers):
        _gpu(kt, vt, kc, vc)
        kv[i] = KVLayer(kt.data_ptr(), vt.data_ptr(), kc.data_ptr(), vc.data_ptr())
        Hkv, D, kv_dt, T = kc.shape[1], kc.shape[3], _dt(kc), kt.shape[2]
    gd = (GDNLayer * max(1, len(gdn_layers)))()
    H = dk = dv = C = 1
    W = 2
    act_dt = DDT_BF16
    for i, (Ssc, S, csc, cst) in enumerate(gdn_layers):
        _gpu(Ssc, S, csc, cst)
        gd[i] = GDNLayer(Ssc.data_ptr(), S.data_ptr(), csc.data_ptr(), cst.data_ptr())
        H, dv, dk = S.shape[1], S.shape[2], S.shape[3]
        W, C, act_dt, T = cst.shape[1] + 1, cst.shape[2], _dt(cst), Ssc.shape[1]
    if B is None:
        if T is None:
            raise ValueError("commit needs B when no layer is given")
        B = T - 1
    if block_table is not None:
        _gpu(block_table)
        if len(kv_layers):
            ps, num_pages = kv_layers[0][2].shape[2], kv_layers[0][2].shape[0]
            if page_size is not None and page_size != ps:
                raise ValueError("commit: page_size %d does not match the page pool's %d" % (page_size, ps))
        elif page_size is None:
            raise ValueError("commit: with no KV layer, give page_size (the capacity is max_blocks * page_size)")
        else:
            ps, num_pages = page_size, 1
        _check("ddt_commit_paged", lib().ddt_commit_paged(
            _ptr(acc_rows), _ptr(acc_len), _ptr(prefix_len), kv, len(kv_layers), Hkv, D, _ptr(block_table),
            block_table.shape[1], ps, num_pages, kv_dt, gd, len(gdn_layers), H, dk, dv, C, W, act_dt, n, B,
            Lp1 - 1, _stream(dev)))
        return
    if len(kv_layers):
        if Pmax is not None and Pmax != kv_layers[0][2].shape[2]:
            raise ValueError("commit: Pmax %d does not match the cache's %d rows" % (Pmax, kv_layers[0][2].shape[2]))
        Pmax = kv_layers[0][2].shape[2]
    elif Pmax is None:
        raise ValueError("commit: with no KV layer, give Pmax (the prefix capacity that guards overflow)")
    _check("ddt_commit", lib().ddt_commit(
        _ptr(acc_rows), _ptr(acc_len), _ptr(prefix_len), kv, len(kv_layers), Hkv, D, Pmax, kv_dt,
        gd, len(gdn_layers), H, dk, dv, C, W, act_dt, n, B, Lp1 - 1, _stream(dev)))


def gdn_replay(acc_rows, acc_len, layers, B):
    """Advance committed GDN/conv state along the accepted path (after commit of the round).
    layers: sequence of (x, conv_w, v, beta, g, S, conv_state) of each GDN layer."""
    _gpu(acc_rows, acc_len)
    n, Lp1 = acc_rows.shape
    dev = acc_rows.device
    tab = (GDNReplayLayer * max(1, len(layers)))()
    H = dk = dv = 1
    C, W, act_dt = 2, 2, DDT_BF16
    for i, (x, cw, v, beta, g, S, cst) in enumerate(layers):
        _gpu(x, cw, v, beta, g, S, cst)
        tab[i] = GDNReplayLayer(x.data_ptr(), cw.data_ptr(), v.data_ptr(), beta.data_ptr(), g.data_ptr(),
                                S.data_ptr(), cst.data_ptr())
        H, dv, dk = S.shape[1], S.shape[2], S.shape[3]
        C, W, act_dt = x.shape[2], cw.shape[1], _dt(x)
    _check("ddt_gdn_replay", lib().ddt_gdn_replay(
        _ptr(acc_rows), _ptr(acc_len), tab, len(layers), H, dk, dv, C, W, act_dt, n, B, Lp1 - 1, _stream(dev)))
