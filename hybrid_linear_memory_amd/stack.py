"""A model-shaped stack of attention layers for streaming video generation.

The summary's hybrid model replaces a fraction (50% or 75%) of a 30-layer
model's softmax attention layers with ARL2 layers ("Attend Locally, Remember
Linearly" technical summary, §3 layer selection and §4 efficiency); the layers
not replaced keep softmax attention over a KV cache that grows by one frame's
keys and values per generated block (§1). This module drives such a stack:
``Arl2Layer`` for the replaced layers, ``SoftmaxCacheLayer`` for the others,
every attention step running in the library's kernels (the cache append is a
device copy).

Only attention is modelled: no projections, MLPs or VAE, and every layer takes
its own inputs, so the stack measures how the attention state and the
attention time grow with the number of generated frames.
"""
from __future__ import annotations

import torch

from . import arl2
from .layer import Arl2Layer


class SoftmaxCacheLayer:
    """Softmax attention of one layer with a KV cache: every pass of frame n
    attends over the clean-pass keys/values of frames 0..n-1 and its own; the
    clean pass's keys/values stay in the cache.

    ``cache`` optionally supplies (k_cache, v_cache) [B, H, max_frames * T, D]
    buffers (several layers may share them when only timing matters)."""

    def __init__(self, shape: arl2.Shape, max_frames: int, device=None, cache=None):
        self.shape = shape
        self.device = torch.device(device or "cuda")
        self.max_frames = max_frames
        cap = max_frames * shape.T
        if cache is None:
            dims = (shape.B, shape.H, cap, shape.D)
            cache = (torch.zeros(dims, dtype=shape.torch_dtype, device=self.device),
                     torch.zeros(dims, dtype=shape.torch_dtype, device=self.device))
        self.k_cache, self.v_cache = cache
        if self.k_cache.shape[2] < cap:
            raise ValueError("cache shorter than max_frames * T")
        self.frame = 0

    def cache_bytes(self, frames: int | None = None) -> int:
        """Bytes the layer's cache holds with `frames` committed frames in it
        (default: the frames committed so far)."""
        s = self.shape
        n = self.frame if frames is None else frames
        return 2 * n * s.T * s.B * s.H * s.D * (2 if s.act_dtype == arl2.BF16 else 4)

    def new_output(self):
        s = self.shape
        return torch.empty((s.B, s.H, s.T, s.D), dtype=s.torch_dtype, device=self.device)

    def _attend(self, q, k, v, o, stream):
        if self.frame >= self.max_frames:
            raise RuntimeError("KV cache full")
        T = self.shape.T
        sl = slice(self.frame * T, (self.frame + 1) * T)
        self.k_cache[:, :, sl].copy_(k)
        self.v_cache[:, :, sl].copy_(v)
        arl2.fullkv_attn(self.shape, q, self.k_cache, self.v_cache, (self.frame + 1) * T, o,
                         stream)
        return o

    def read(self, q, k, v, o=None, stream=None):
        return self._attend(q, k, v, self.new_output() if o is None else o, stream)

    def clean_pass(self, q, k, v, beta=None, alpha=None, o=None, stream=None):
        o = self._attend(q, k, v, self.new_output() if o is None else o, stream)
        self.frame += 1
        return o


class HybridStack:
    """Layers l with mask[l] true are ARL2 layers (phis[l] = (phi_q, phi_k,
    phi_v)), the others softmax layers with a KV cache of max_frames frames.
    With ``shared_cache`` the softmax layers share one cache buffer (their
    work is unchanged; only for timing, the values then mix)."""

    def __init__(self, shape: arl2.Shape, mask, phis, max_frames: int, device=None,
                 shared_cache: bool = False):
        self.shape = shape
        self.mask = [bool(m) for m in mask]
        dev = torch.device(device or "cuda")
        cache = None
        if shared_cache and not all(self.mask):
            dims = (shape.B, shape.H, max_frames * shape.T, shape.D)
            cache = (torch.zeros(dims, dtype=shape.torch_dtype, device=dev),
                     torch.zeros(dims, dtype=shape.torch_dtype, device=dev))
        self.layers = []
        for l, is_arl2 in enumerate(self.mask):
            if is_arl2:
                self.layers.append(Arl2Layer(shape, *phis[l], device=dev))
            else:
                self.layers.append(SoftmaxCacheLayer(shape, max_frames, dev, cache))

    def read(self, inputs, outs=None):
        """A denoising pass through every layer: inputs[l] = (q, k, v)."""
        return [lay.read(*inputs[l], o=None if outs is None else outs[l])
                for l, lay in enumerate(self.layers)]

    def clean_pass(self, inputs, gates, outs=None):
        """The clean pass: inputs[l] = (q, k, v), gates[l] = (beta, alpha)
        (used by the ARL2 layers)."""
        return [lay.clean_pass(*inputs[l], *gates[l], o=None if outs is None else outs[l])
                for l, lay in enumerate(self.layers)]

    def state_bytes(self, frames: int | None = None) -> int:
        """Attention state the stack holds: the softmax layers' caches (after
        `frames` frames, default their current fill) plus every ARL2 layer's
        double-buffered state and prepared map."""
        s = self.shape
        arl2_bytes = 2 * s.B * s.H * s.D * s.D * 4 + 2 * arl2.prepared_bytes(s)
        total = 0
        for lay, is_arl2 in zip(self.layers, self.mask):
            total += arl2_bytes if is_arl2 else lay.cache_bytes(frames)
        return total
