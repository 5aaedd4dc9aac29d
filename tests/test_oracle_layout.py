"""Pins of the coarse-key bytes and of the cache-layout accounting.

The 890 bytes/token global-KV figure is printed in the paper notes (Figure 1 caption) and
in the Chinese reading's summary.  Reading used here: main KV = 512 E2M1 values + one E4M3
scale per 16 channels (288 B, "FP4 Main KV Cache" / 3.5), indexer key = 64 E4M3 values +
a 4-byte scale (68 B); encoder Full layers store one entry per 2 tokens, the decoder Full
layer one per token (3.3 / "Model Setup Numbers"), Reindex/Reuse layers store nothing.
"""
import json
import os

import numpy as np
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def test_global_kv_bytes_per_token_reproduces_890():
    g = json.load(open(GOLDEN))
    main = g["main_kv_dim"] * g["main_kv_bits"] // 8 + g["main_kv_dim"] // g["main_kv_channels_per_scale"] * \
        g["main_kv_scale_bytes"]
    index_key = 64 + 4
    per_entry = main + index_key
    enc_full = g["encoder_csa2_groups"]            # one Full layer per encoder group
    dec_full = 1                                   # only the first decoder group starts with Full
    entries_per_token = enc_full / g["encoder_compression"] + dec_full / g["decoder_compression"]
    assert main == 288 and per_entry == 356
    assert entries_per_token * per_entry == g["global_kv_bytes_per_token"]
    assert g["pool_blocks"] * g["pool_block_size"] == g["pool_candidates"]


def test_coarse_keys_bytes_against_sequential_fp32_mean():
    wl = workloads.workload("hier1m", N=200)
    k = wl.index_keys(0)[None]
    k8, ks = oracle.quantize_fp8(k)
    nk = np.array([200], np.int32)
    kb8, kbs = oracle.coarse_keys(k8, ks, nk, 64)
    dec = torch.from_numpy(k8[0]).view(torch.float8_e4m3fn).double().numpy()
    vals = (dec * ks[0][:, None].astype(np.float64)).astype(np.float32)     # fl32(sk * key)
    for blk in range(4):
        rows = vals[blk * 64:min(200, blk * 64 + 64)]
        mean = np.zeros(64, np.float32)
        for c in range(64):
            acc = np.float32(0)
            for r in rows[:, c]:
                acc = np.float32(acc + r)
            mean[c] = np.float32(acc / np.float32(len(rows)))
        s = np.float32(np.abs(mean).max() / np.float32(448))
        ref = torch.from_numpy((mean / s).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert kbs[0, blk] == s
        assert np.array_equal(kb8[0, blk], ref)
