"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and builds input structure only; it holds none
of the dequantize-and-multiply arithmetic and none of the quantizers.  Every
array comes from ``numpy.random.default_rng(crc32(tag))`` so a tag names an
input reproducibly on any host.

Workloads it stands in for (shapes and value distributions only; no trained
weights or datasets are used):
* weights W [N, K] ~ N(0, 0.02^2) in fp32, activations ~ N(0, 1);
* act-order: a random permutation pi of the K input columns, grouped in sorted
  order: g_idx[pi[j]] = j // G  (GPTQ ``desc_act`` / ``--act-order``,
  [P2] §三 3.1, [P4] "技术原理" section);
* AWQ per-input-channel scales s ~ U[0.5, 2] folded as W * s and x / s, all
  4-bit, no mixed precision ([P3] §4.1);
* prefill activations with 1 % of input channels multiplied by 20 (outlier
  channels, the reason AWQ protects salient channels, [P3] §4.1).
"""

import zlib

import numpy as np
import torch


def rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def weights(tag, N, K, std=0.02):
    return rng(tag).standard_normal((N, K), dtype=np.float32) * np.float32(std)


def activations(tag, M, K):
    return rng(tag).standard_normal((M, K), dtype=np.float32)


def to_f16_bits(x32):
    return np.asarray(x32, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_bits(x32, dtype):
    return to_f16_bits(x32) if dtype == "f16" else to_bf16_bits(x32)


def act_order_gidx(tag, K, group_size=128):
    pi = rng(tag).permutation(K)
    g = np.empty(K, dtype=np.int32)
    g[pi] = (np.arange(K) // group_size).astype(np.int32)
    return g


def awq_scales(tag, K):
    return rng(tag).uniform(0.5, 2.0, size=K).astype(np.float32)


def awq_fold(W, x32, s):
    """Fold per-input-channel scales: W' = fp32(W * s), x' = fp32(x / s)."""
    s = np.asarray(s, dtype=np.float32)
    return (W * s[None, :]).astype(np.float32), (x32 / s[None, :]).astype(np.float32)


def outlier_channels(tag, K, frac=0.01):
    n = int(round(frac * K))
    return np.sort(rng(tag).choice(K, size=n, replace=False))


def with_outliers(x32, channels, factor=20.0):
    y = np.array(x32, dtype=np.float32, copy=True)
    y[:, channels] *= np.float32(factor)
    return y
