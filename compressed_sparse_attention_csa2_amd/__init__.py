"""CSA2 (Compressed Sparse Attention 2) decode / chunked-prefill hot path for MI355X.

Thin ctypes binding over ``libcsa2.so`` (hand-written HIP kernels for gfx950, C ABI in
``include/csa2.h``).  Every step runs in the library's kernels; this module only checks
tensor dtypes/shapes, passes ``data_ptr()``s and the current HIP stream, allocates
workspaces with torch, and turns a non-zero status into :class:`Csa2Error`.  There is
no CPU fallback: without the built library every call raises.

Method (see the header for per-call definitions): per query row an indexer scores the
cached entries, the Top-K are selected (ties to the lower position), the FP4 E2M1 main
KV rows are gathered and dequantised, and softmax attention runs over those rows only;
Full / Reindex / Reuse layers share the cache and (Reuse) the selected indices.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

# enums of include/csa2.h
OK = 0
F32, BF16 = 0, 1
FMT_FP4_PER_CHANNEL, FMT_FP8_PER_TOKEN, FMT_FP4_G16, FMT_FP4_PER_TOKEN = 0, 1, 2, 3
SCALE_COMPUTE, SCALE_GIVEN = 0, 1
PREC_FP32, PREC_FP8, PREC_FP4 = 0, 1, 2
FULL, REINDEX, REUSE = 0, 1, 2
MODE_NAMES = {"full": FULL, "reindex": REINDEX, "reuse": REUSE}

EXPORTS = [
    "csa2_status_string", "csa2_device_check", "csa2_quantize_kv", "csa2_gather_dequant", "csa2_index_score",
    "csa2_index_score_workspace_size", "csa2_topk", "csa2_topk_workspace_size", "csa2_index_topk",
    "csa2_index_topk_workspace_size", "csa2_sparse_attend", "csa2_sparse_attend_workspace_size",
    "csa2_layer_group", "csa2_layer_group_workspace_size", "csa2_coarse_keys", "csa2_hier_select",
    "csa2_hier_select_workspace_size", "csa2_layer_group_noalloc", "csa2_stream_probe",
]

# bytes of the library-held scratch array of csa2_layer_group_noalloc (one per GPU)
NOALLOC_SCRATCH_BYTES = 64 << 20


class Csa2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, status_string(status)))


class _Swa(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("n_max", ctypes.c_int64),
                ("end", ctypes.c_void_p), ("window", ctypes.c_int)]


class _Layer(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("q_idx", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("q_attn", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("pool", ctypes.c_void_p), ("swa", ctypes.POINTER(_Swa))]


class _GroupCache(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int), ("Hq", ctypes.c_int),
                ("D", ctypes.c_int), ("K", ctypes.c_int), ("n_max", ctypes.c_int64), ("n_keys", ctypes.c_void_p),
                ("kv_codes", ctypes.c_void_p), ("kv_scales", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("prec", ctypes.c_int), ("q_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int), ("softmax_scale", ctypes.c_float), ("pool_block", ctypes.c_int),
                ("pool_blocks", ctypes.c_int), ("kv_fmt", ctypes.c_int), ("window", ctypes.c_int),
                ("T", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcsa2.so is not built (%s); run "
                               "`python -m compressed_sparse_attention_csa2_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        i, i64, f, p, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        sig = {
            "csa2_status_string": ([i], ctypes.c_char_p),
            "csa2_device_check": ([], i),
            "csa2_quantize_kv": ([i, i, i, i, i, p, i, i64, i64, p, i64, p, p, p], i),
            "csa2_gather_dequant": ([i, i, i, i, i, p, p, i64, p, p, p], i),
            "csa2_index_score": ([i, i, i, i, i, p, i, p, p, p, i64, p, p, p, i, p, p, sz, p], i),
            "csa2_index_score_workspace_size": ([i, i, i64], sz),
            "csa2_topk": ([i, i, i64, p, p, i, p, p, p, sz, p], i),
            "csa2_topk_workspace_size": ([i, i, i64, i], sz),
            "csa2_index_topk": ([i, i, i, i, i, p, i, p, p, p, i64, p, p, p, i, i, p, p, p, sz, p], i),
            "csa2_index_topk_workspace_size": ([i, i, i64, i], sz),
            "csa2_sparse_attend": ([i, i, i, i, p, i, i, p, p, i64, p, i, p, f, p, i, p, p, sz, p], i),
            "csa2_sparse_attend_workspace_size": ([i, i, i, i, i, i, i], sz),
            "csa2_layer_group": ([p, i, p, p, sz, p], i),
            "csa2_layer_group_workspace_size": ([p, i], sz),
            "csa2_layer_group_noalloc": ([p, i, p, p], i),
            "csa2_stream_probe": ([p, i64, i, p, p], i),
            "csa2_coarse_keys": ([i, i64, p, i, i, p, p, p, p, p], i),
            "csa2_hier_select": ([i, i, i, p, i, p, p, p, p, p, i64, p, i, i, i, p, p, p, sz, p], i),
            "csa2_hier_select_workspace_size": ([i, i64, i, i, i], sz),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().csa2_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise Csa2Error(status, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError("unsupported dtype %s" % t.dtype)


_ws_cache: dict = {}


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A device byte buffer of at least nbytes, one per (device, stream): calls on one
    stream are ordered, so they may share it; a buffer that grows is released to torch's
    allocator, which hands it out again only in that stream's order."""
    if nbytes == 0:
        return None
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def device_check() -> int:
    return lib().csa2_device_check()


# ------------------------------------------------------------------------------ write side
def quantize_kv(fmt: int, x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                scale_policy: int = SCALE_COMPUTE, n0: Optional[torch.Tensor] = None) -> None:
    """x [B][T][D] (fp32/bf16; the row stride may exceed D) -> codes/scales (see csa2.h)."""
    B, T, D = x.shape
    if x.stride(2) != 1:
        raise ValueError("x must have a contiguous last dimension")
    n_max = codes.shape[1]
    _check(lib().csa2_quantize_kv(fmt, scale_policy, B, T, D, x.data_ptr(), _dtype_code(x), x.stride(0),
                                  x.stride(1), _ptr(n0), n_max, _ptr(codes), _ptr(scales), _stream()),
           "csa2_quantize_kv")


def kv_format(scales: torch.Tensor) -> int:
    """The main-KV layout a scales tensor belongs to: uint8 [B][n_max][D/16] E4M3 bytes is
    the per-16-channel layout (FMT_FP4_G16), fp32 [B][D] the per-channel one."""
    return FMT_FP4_G16 if scales.dtype == torch.uint8 else FMT_FP4_PER_CHANNEL


def gather_dequant(codes: torch.Tensor, scales: torch.Tensor, idx: torch.Tensor,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    B, n_max, Dh = codes.shape
    _, T, K = idx.shape
    if out is None:
        out = torch.empty((B, T, K, 2 * Dh), dtype=torch.float32, device=codes.device)
    _check(lib().csa2_gather_dequant(kv_format(scales), B, T, K, 2 * Dh, _ptr(codes), _ptr(scales), n_max, _ptr(idx),
                                     _ptr(out), _stream()), "csa2_gather_dequant")
    return out


# ------------------------------------------------------------------------------ indexer
def index_score(prec: int, q: torch.Tensor, w: torch.Tensor, k: torch.Tensor, k_scale: Optional[torch.Tensor],
                n_keys: torch.Tensor, q_limit: Optional[torch.Tensor] = None, cand: Optional[torch.Tensor] = None,
                scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    B, T, H, dk = q.shape
    n_max = k.shape[1]
    C = 0 if cand is None else cand.shape[-1]
    ncols = C if cand is not None else n_max
    if scores is None:
        scores = torch.empty((B, T, ncols), dtype=torch.float32, device=q.device)
    nb = lib().csa2_index_score_workspace_size(B, T, ncols)
    ws = _workspace(nb, q.device)
    _check(lib().csa2_index_score(prec, B, T, H, dk, _ptr(q), _dtype_code(q), _ptr(w), _ptr(k), _ptr(k_scale),
                                  n_max, _ptr(n_keys), _ptr(q_limit), _ptr(cand), C, _ptr(scores), _ptr(ws), nb,
                                  _stream()), "csa2_index_score")
    return scores


def topk(scores: torch.Tensor, K: int, cand: Optional[torch.Tensor] = None, want_values: bool = False):
    B, T, ncols = scores.shape
    idx = torch.empty((B, T, K), dtype=torch.int32, device=scores.device)
    val = torch.empty((B, T, K), dtype=torch.float32, device=scores.device) if want_values else None
    nb = lib().csa2_topk_workspace_size(B, T, ncols, K)
    ws = _workspace(nb, scores.device)
    _check(lib().csa2_topk(B, T, ncols, _ptr(scores), _ptr(cand), K, _ptr(idx), _ptr(val), _ptr(ws), nb,
                           _stream()), "csa2_topk")
    return (idx, val) if want_values else idx


def index_topk(prec: int, q: torch.Tensor, w: torch.Tensor, k: torch.Tensor, k_scale: Optional[torch.Tensor],
               n_keys: torch.Tensor, K: int, q_limit: Optional[torch.Tensor] = None,
               cand: Optional[torch.Tensor] = None, want_values: bool = False, idx: Optional[torch.Tensor] = None):
    B, T, H, dk = q.shape
    n_max = k.shape[1]
    C = 0 if cand is None else cand.shape[-1]
    ncols = C if cand is not None else n_max
    if idx is None:
        idx = torch.empty((B, T, K), dtype=torch.int32, device=q.device)
    val = torch.empty((B, T, K), dtype=torch.float32, device=q.device) if want_values else None
    nb = lib().csa2_index_topk_workspace_size(B, T, ncols, K)
    ws = _workspace(nb, q.device)
    _check(lib().csa2_index_topk(prec, B, T, H, dk, _ptr(q), _dtype_code(q), _ptr(w), _ptr(k), _ptr(k_scale), n_max,
                                 _ptr(n_keys), _ptr(q_limit), _ptr(cand), C, K, _ptr(idx), _ptr(val), _ptr(ws), nb,
                                 _stream()), "csa2_index_topk")
    return (idx, val) if want_values else idx


# ------------------------------------------------------------------------------ attention
class Swa:
    """A layer's own sliding-window cache: codes [B][n_max][D] uint8 (E4M3) and scales
    [B][n_max] fp32 (as quantize_kv writes them with FMT_FP8_PER_TOKEN), end [B][T] int32:
    query row (b, t) attends to rows [max(0, end - window), end)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, end: torch.Tensor, window: int):
        self.codes, self.scales, self.end, self.window = codes, scales, end, int(window)

    def struct(self) -> _Swa:
        return _Swa(_ptr(self.codes), _ptr(self.scales), self.codes.shape[1], _ptr(self.end), self.window)


def sparse_attend(q: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, idx: torch.Tensor,
                  softmax_scale: float, out_dtype: Optional[torch.dtype] = None, want_lse: bool = True,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  swa: Optional[Swa] = None):
    B, T, Hq, D = q.shape
    n_max = codes.shape[1]
    K = idx.shape[-1]
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    qd = _dtype_code(q)
    nb = lib().csa2_sparse_attend_workspace_size(B, T, Hq, D, K, qd, swa.window if swa else 0)
    ws = _workspace(nb, q.device)
    sw = swa.struct() if swa else None
    _check(lib().csa2_sparse_attend(B, T, Hq, D, _ptr(q), qd, kv_format(scales), _ptr(codes), _ptr(scales), n_max,
                                    _ptr(idx), K, ctypes.byref(sw) if sw else None, float(softmax_scale), _ptr(out),
                                    _dtype_code(out), _ptr(lse), _ptr(ws), nb, _stream()), "csa2_sparse_attend")
    return out, lse


# ------------------------------------------------------------------------------ layer group
class GroupCache:
    """The shared cache of a layer group (all device tensors).  kv_scales: fp32 [B][D]
    (one scale per channel) or uint8 [B][n_max][D/16] (one E4M3 scale per 16 channels of
    each entry)."""

    def __init__(self, n_keys, kv_codes, kv_scales, k, k_scale, K, softmax_scale, prec=PREC_FP8, pool=None):
        """pool: None, or (block, blocks): Full layers leave the positions of their `blocks`
        best blocks of `block` positions (by block maximum) to the later Reindex layers."""
        self.n_keys, self.kv_codes, self.kv_scales, self.k, self.k_scale = n_keys, kv_codes, kv_scales, k, k_scale
        self.K, self.softmax_scale, self.prec = K, softmax_scale, prec
        self.pool = pool

    def struct(self, H, dk, Hq, q_dtype, out_dtype, window=0, T=1):
        B, n_max, Dh = self.kv_codes.shape
        pb, pn = self.pool if self.pool else (0, 0)
        return _GroupCache(B, H, dk, Hq, 2 * Dh, self.K, n_max, _ptr(self.n_keys), _ptr(self.kv_codes),
                           _ptr(self.kv_scales), _ptr(self.k), _ptr(self.k_scale), self.prec, q_dtype, out_dtype,
                           float(self.softmax_scale), pb, pn, kv_format(self.kv_scales), window, T)


class GroupPlan:
    """A layer group with every argument marshalled once; run() is one C-ABI call."""

    def __init__(self, layers: Sequence[dict], cache: GroupCache, out_dtype: Optional[torch.dtype] = None):
        self.layers = list(layers)
        self._arr, self._gc, self._ws, self._nb, self._swa = _marshal_group(self.layers, cache, out_dtype)

    def run(self):
        _check(lib().csa2_layer_group(self._arr, len(self.layers), ctypes.byref(self._gc), _ptr(self._ws), self._nb,
                                      _stream()), "csa2_layer_group")
        return self.layers


def layer_group(layers: Sequence[dict], cache: GroupCache, out_dtype: Optional[torch.dtype] = None):
    """Run Full/Reindex/Reuse layers in order over one shared cache.

    layers: dicts with mode ('full'|'reindex'|'reuse'), q_idx [B][T][H][dk], w [B][T][H],
    q_attn [B][T][Hq][D] (T query tokens per sequence, 1 for plain decode; with T > 1 their
    own entries are the cache's last T and token t sees positions < n_keys - (T - 1 - t))
    and optionally out, lse, idx tensors, 'swa' (the layer's own
    sliding-window cache, a Swa), and for Full layers of a cache with a pool a 'pool' int32
    tensor [B][blocks*block] that receives the pool's positions.  Returns the layer dicts with 'out', 'lse' and (Full/Reindex) 'idx' filled."""
    return GroupPlan(layers, cache, out_dtype).run()


def layer_group_noalloc(layers: Sequence[dict], cache: GroupCache, out_dtype: Optional[torch.dtype] = None):
    """layer_group through csa2_layer_group_noalloc: the library's own scratch array serves
    as the workspace, so the call itself allocates no device memory (outputs missing from
    the layer dicts are still created here, before the call)."""
    arr, gc, _, _, swas = _marshal_group(layers, cache, out_dtype, workspace=False)
    _check(lib().csa2_layer_group_noalloc(arr, len(layers), ctypes.byref(gc), _stream()), "csa2_layer_group_noalloc")
    del swas  # the window structs stay alive until the call has returned
    return layers


def _marshal_group(layers, cache, out_dtype, workspace=True):
    first = layers[0]
    q_attn = first["q_attn"]
    B, T, Hq, D = q_attn.shape
    H, dk = (first["q_idx"].shape[2], first["q_idx"].shape[3]) if first.get("q_idx") is not None else (32, 64)
    odt = out_dtype or q_attn.dtype
    arr = (_Layer * len(layers))()
    swas = [L["swa"].struct() if L.get("swa") is not None else None for L in layers]  # kept alive by the plan
    window = max([sw.window for sw in swas if sw is not None], default=0)
    for i, L in enumerate(layers):
        mode = MODE_NAMES[L["mode"]] if isinstance(L["mode"], str) else int(L["mode"])
        if tuple(L["q_attn"].shape[:2]) != (B, T):
            raise ValueError("every layer's q_attn must be [B][T][Hq][D] with the same B and T")
        if L.get("out") is None:
            L["out"] = torch.empty((B, T, Hq, D), dtype=odt, device=q_attn.device)
        if L.get("lse") is None:
            L["lse"] = torch.empty((B, T, Hq), dtype=torch.float32, device=q_attn.device)
        if mode != REUSE and L.get("idx") is None:
            L["idx"] = torch.empty((B, T, cache.K), dtype=torch.int32, device=q_attn.device)
        p = L.get("pool")
        if p is not None and mode == FULL:
            if not cache.pool:
                raise ValueError("a pool output was given but the cache has no pool")
            if p.dtype != torch.int32 or not p.is_contiguous() or p.numel() != B * T * cache.pool[0] * cache.pool[1]:
                raise ValueError("pool must be a contiguous int32 tensor of B * T * block * blocks elements")
        arr[i] = _Layer(mode, _ptr(L.get("q_idx")), _ptr(L.get("w")), _ptr(L["q_attn"]), _ptr(L["out"]),
                        _ptr(L["lse"]), _ptr(L.get("idx")) if mode != REUSE else None,
                        _ptr(L.get("pool")) if mode == FULL else None,
                        ctypes.pointer(swas[i]) if swas[i] is not None else None)
    qd = _dtype_code(q_attn)
    gc = cache.struct(H, dk, Hq, qd, _dtype_code(torch.empty(0, dtype=odt)), window, T)
    nb = lib().csa2_layer_group_workspace_size(ctypes.byref(gc), len(layers))
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=q_attn.device) if workspace else None
    return arr, gc, ws, nb, swas


# ------------------------------------------------------------------------------ two-level indexer
def coarse_keys(k8: torch.Tensor, k_scale: torch.Tensor, n_keys: torch.Tensor, block: int):
    B, n_max, dk = k8.shape
    nb = (n_max + block - 1) // block
    kb8 = torch.empty((B, nb, dk), dtype=torch.uint8, device=k8.device)
    kbs = torch.empty((B, nb), dtype=torch.float32, device=k8.device)
    _check(lib().csa2_coarse_keys(B, n_max, _ptr(n_keys), dk, block, _ptr(k8), _ptr(k_scale), _ptr(kb8), _ptr(kbs),
                                  _stream()), "csa2_coarse_keys")
    return kb8, kbs


def hier_select(q: torch.Tensor, w: torch.Tensor, k8: torch.Tensor, k_scale: torch.Tensor, kb8: torch.Tensor,
                kb_scale: torch.Tensor, n_keys: torch.Tensor, block: int, block_topk: int, K: int,
                want_blocks: bool = False):
    B, T, H, dk = q.shape
    if T != 1:
        raise ValueError("hier_select is a decode call (one query token per sequence)")
    n_max = k8.shape[1]
    idx = torch.empty((B, 1, K), dtype=torch.int32, device=q.device)
    blk = torch.empty((B, 1, block_topk), dtype=torch.int32, device=q.device) if want_blocks else None
    nb = lib().csa2_hier_select_workspace_size(B, n_max, block, block_topk, K)
    ws = _workspace(nb, q.device)
    _check(lib().csa2_hier_select(B, H, dk, _ptr(q), _dtype_code(q), _ptr(w), _ptr(k8), _ptr(k_scale), _ptr(kb8),
                                  _ptr(kb_scale), n_max, _ptr(n_keys), block, block_topk, K, _ptr(idx), _ptr(blk),
                                  _ptr(ws), nb, _stream()), "csa2_hier_select")
    return (idx, blk) if want_blocks else idx


# ------------------------------------------------------------------------------ measurement
def stream_probe(buf: torch.Tensor, blocks: int = 2048, sink: Optional[torch.Tensor] = None) -> None:
    """One read of the whole of `buf` by the library's streaming probe kernel (a ceiling for
    the key scan's HBM rate; it computes nothing)."""
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    _check(lib().csa2_stream_probe(_ptr(buf), buf.numel() * buf.element_size(), blocks, _ptr(sink), _stream()),
           "csa2_stream_probe")
