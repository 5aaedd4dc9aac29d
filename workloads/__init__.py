"""Seeded synthetic workloads for the CSA2 decode / chunked-prefill path.

This module only draws numbers (no quantisation, scoring, selection or attention): the
GPU path and the CPU oracle each apply the method to the same drawn values.

The workloads follow the shapes the DeepSeek-V4.1-Flash notes give for CSA2 ("Model Setup
Numbers": 32 indexer heads, Top-512, 64 attention heads of dim 512; "FP4 Main KV Cache":
512-dim E2M1 entries) and the five synthetic configurations this library is measured on:

* ``tiny``      Full-mode decode, B=1, N=4096, fp32 indexer 4x64, K=64, D=128, 8 heads fp32.
* ``full64k``   Full-mode decode, B=16, N=65536, fp8 indexer 32x64, K=512, D=512, 64 heads bf16,
                main KV N(0,1) with 1 % of channels (5 of 512) scaled by 8.
* ``group128k`` Full -> Reindex -> Reuse, B=16, N=131072, shapes as ``full64k``; each layer draws
                its own indexer query, head weights and attention query.
* ``hier1m``    two-level indexer decode, B=1, N=2^20, coarse blocks of 64, top-256 blocks,
                K=1024, no outliers.
* ``prefill``   chunked prefill, B=1, 262144 cached entries + 4096 new tokens, causal, K=512.

Value recipe: indexer keys, indexer queries, attention queries and main-KV rows ~ N(0,1);
head weights ~ U(0,1); bf16 tensors are N(0,1) fp32 values rounded to nearest-even bf16.
Streams are SplitMix64 counter-based (one per tensor id), normals by Box-Muller in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libcsa2_workloads.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the generator with gcc (fp-contract off so bytes never depend on flags)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float
        p = ctypes.c_void_p
        lib.wl_u64.argtypes = [u64, u64, u64]
        lib.wl_u64.restype = u64
        lib.wl_uniform_f32.argtypes = [u64, u64, i64, i64, f32, f32, p]
        lib.wl_normal_f32.argtypes = [u64, u64, i64, i64, p]
        lib.wl_round_bf16.argtypes = [p, i64]
        lib.wl_scale_channels.argtypes = [p, i64, ctypes.c_int, p, ctypes.c_int, f32]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(seed: int, stream: int, shape, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().wl_normal_f32(seed, stream, offset, out.size, _ptr(out))
    return out


def uniform(seed: int, stream: int, shape, lo: float = 0.0, hi: float = 1.0, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().wl_uniform_f32(seed, stream, offset, out.size, lo, hi, _ptr(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16-representable fp32 values (nearest-even), in place."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    _load().wl_round_bf16(_ptr(x), x.size)
    return x


def u64(seed: int, stream: int, i: int) -> int:
    return int(_load().wl_u64(seed, stream, i))


def scale_channels(x: np.ndarray, channels, factor: float) -> np.ndarray:
    ch = np.ascontiguousarray(np.asarray(channels, dtype=np.int32))
    rows = x.size // x.shape[-1]
    _load().wl_scale_channels(_ptr(x), rows, x.shape[-1], _ptr(ch), ch.size, factor)
    return x


def pick_channels(seed: int, stream: int, dim: int, count: int) -> np.ndarray:
    """`count` distinct channels of `dim`, by a seeded partial Fisher-Yates shuffle, sorted."""
    perm = list(range(dim))
    for i in range(count):
        j = i + u64(seed, stream, i) % (dim - i)
        perm[i], perm[j] = perm[j], perm[i]
    return np.array(sorted(perm[:count]), dtype=np.int32)


# Stream ids (one per tensor; per-layer tensors add 16 * layer).
S_KV = 1          # main-KV rows, fp32 N(0,1)
S_IDXK = 2        # indexer keys, fp32 N(0,1)
S_OUTLIER = 3     # choice of outlier channels
S_KV_NEW = 4      # prefill: new tokens' main-KV rows (bf16)
S_IDXK_NEW = 5    # prefill: new tokens' indexer keys
S_Q_IDX = 16      # + 16*layer: indexer query
S_W = 17          # + 16*layer: head weights
S_Q_ATTN = 18     # + 16*layer: attention query


@dataclass
class Workload:
    """Shapes and value recipe of one synthetic configuration."""
    name: str
    seed: int
    B: int
    N: int                      # cached entries per sequence (decode) / already cached (prefill)
    T: int = 1                  # query tokens per sequence
    H: int = 32                 # indexer heads
    dk: int = 64                # indexer dim
    K: int = 512                # Top-K
    D: int = 512                # main-KV dim
    Hq: int = 64                # attention heads
    index_fp8: bool = True      # indexer keys E4M3 per token + bf16 queries (else fp32 throughout)
    attn_bf16: bool = True      # attention query / output bf16 (else fp32)
    outlier_frac: float = 0.0   # fraction of main-KV channels scaled by `outlier_factor`
    outlier_factor: float = 8.0
    modes: tuple = ("full",)    # layer modes of the group
    coarse_block: int = 0       # two-level indexer: entries per coarse block (0 = flat)
    coarse_topk: int = 0        # two-level indexer: blocks kept
    prefill: bool = False       # chunked prefill: T new tokens appended after N cached ones
    extra: dict = field(default_factory=dict)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def n_max(self) -> int:
        return self.N + (self.T if self.prefill else 0)

    def outlier_channels(self) -> np.ndarray:
        n = int(np.floor(self.outlier_frac * self.D))
        if n == 0:
            return np.zeros(0, dtype=np.int32)
        return pick_channels(self.seed, S_OUTLIER, self.D, n)

    # ---- drawn tensors (fp32 numpy arrays holding the values the method sees) ----
    def main_kv(self, b: int, rows: int | None = None, row0: int = 0) -> np.ndarray:
        """Cached main-KV rows [rows][D] of sequence b (before FP4 quantisation)."""
        rows = self.N if rows is None else rows
        x = normal(self.seed, S_KV, (rows, self.D), offset=(b * self.N + row0) * self.D)
        ch = self.outlier_channels()
        if ch.size:
            scale_channels(x, ch, self.outlier_factor)
        return x

    def index_keys(self, b: int, rows: int | None = None, row0: int = 0) -> np.ndarray:
        """Cached indexer keys [rows][dk] of sequence b (fp32, before E4M3 quantisation)."""
        rows = self.N if rows is None else rows
        return normal(self.seed, S_IDXK, (rows, self.dk), offset=(b * self.N + row0) * self.dk)

    def new_kv(self) -> np.ndarray:
        """Prefill: the T new tokens' main-KV rows [B][T][D], bf16 values."""
        return round_bf16(normal(self.seed, S_KV_NEW, (self.B, self.T, self.D)))

    def new_index_keys(self) -> np.ndarray:
        """Prefill: the T new tokens' indexer keys [B][T][dk], fp32."""
        return normal(self.seed, S_IDXK_NEW, (self.B, self.T, self.dk))

    def index_query(self, layer: int = 0) -> np.ndarray:
        q = normal(self.seed, S_Q_IDX + 16 * layer, (self.B, self.T, self.H, self.dk))
        return round_bf16(q) if self.index_fp8 else q

    def head_weights(self, layer: int = 0) -> np.ndarray:
        return uniform(self.seed, S_W + 16 * layer, (self.B, self.T, self.H))

    def attn_query(self, layer: int = 0) -> np.ndarray:
        q = normal(self.seed, S_Q_ATTN + 16 * layer, (self.B, self.T, self.Hq, self.D))
        return round_bf16(q) if self.attn_bf16 else q


WORKLOADS = {
    "tiny": Workload("tiny", seed=0, B=1, N=4096, H=4, dk=64, K=64, D=128, Hq=8,
                     index_fp8=False, attn_bf16=False),
    "full64k": Workload("full64k", seed=1, B=16, N=65536, outlier_frac=0.01),
    "group128k": Workload("group128k", seed=2, B=16, N=131072, outlier_frac=0.01,
                          modes=("full", "reindex", "reuse")),
    "hier1m": Workload("hier1m", seed=3, B=1, N=1 << 20, K=1024, coarse_block=64, coarse_topk=256),
    "prefill": Workload("prefill", seed=4, B=1, N=262144, T=4096, prefill=True),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with some fields overridden (smaller parity cases)."""
    import dataclasses
    return dataclasses.replace(WORKLOADS[name], **overrides)
