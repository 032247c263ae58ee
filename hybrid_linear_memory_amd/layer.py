"""Streaming driver of one ARL2 hybrid attention layer.

Holds the double-buffered fp32 state, the feature maps and the workspace,
and enforces the pass order of the memory-state management rules
("Attend Locally, Remember Linearly" technical summary, §2.2): within a
frame every denoising read and the clean pass see the same S_{N-1}; the
state is written once, by the clean pass, into the other buffer; the
buffers swap and the frame index advances only then.

The pass order itself (``PassSequencer``) is plain host logic with no device
dependency.
"""
from __future__ import annotations

import torch

from . import arl2


class SequenceError(RuntimeError):
    """A pass was issued out of the read* -> clean pass order."""


class NonFiniteInput(ValueError):
    """An input of a pass holds a NaN or an infinity (debug check)."""


def check_finite(**tensors):
    """Raise NonFiniteInput naming the first given tensor that holds a NaN or
    an infinity (None entries are skipped). Reads every element, and on a
    device tensor waits for the stream: a debug aid, off by default."""
    for name, t in tensors.items():
        if t is not None and not bool(torch.isfinite(t).all()):
            raise NonFiniteInput(f"{name} holds non-finite values")


class PassSequencer:
    """Frame / pass bookkeeping. With ``n_denoise`` set (strict mode) each
    frame must have exactly that many reads before its clean pass."""

    def __init__(self, n_denoise: int | None = None):
        if n_denoise is not None and n_denoise < 0:
            raise ValueError("n_denoise must be >= 0")
        self.n_denoise = n_denoise
        self.frame = 0
        self.reads = 0

    def before_read(self):
        if self.n_denoise is not None and self.reads >= self.n_denoise:
            raise SequenceError(
                f"frame {self.frame}: {self.reads} denoising reads already issued; the next "
                "pass of this frame must be the clean pass")

    def after_read(self):
        self.reads += 1

    def before_clean_pass(self):
        if self.n_denoise is not None and self.reads != self.n_denoise:
            raise SequenceError(
                f"frame {self.frame}: clean pass after {self.reads} reads, expected "
                f"{self.n_denoise}")

    def after_clean_pass(self):
        self.frame += 1
        self.reads = 0

    def restore(self, frame: int):
        if frame < 0:
            raise ValueError("frame index must be >= 0")
        self.frame = frame
        self.reads = 0


class Arl2Layer:
    """One hybrid attention layer over B streams on the current device.

    phi_q, phi_k, phi_v: [H, D, D] tensors of the activation dtype.

    With prepared reads (the default) the clean pass is one library call
    (arl2_clean_pass_prepared: read and commit in one launch on bf16 shapes);
    ``fused_clean=False`` issues the read and the commit as two calls instead.

    ``access="token"`` runs the ablated alternative to frame-level access
    (the summary's §4): within each pass token t reads the state updated by
    the frame's earlier tokens (arl2_token_read / arl2_token_clean_pass); the
    state is still written once per frame, by the clean pass.

    ``check_finite=True`` (debug) checks every input of a pass for NaN and
    infinity before anything is launched and raises NonFiniteInput, leaving
    the state and the pass order untouched.
    """

    def __init__(self, shape: arl2.Shape, phi_q, phi_k, phi_v, n_denoise: int | None = None,
                 device=None, prepared: bool = True, fused_clean: bool = True,
                 access: str = "frame", check_finite: bool = False):
        if access not in ("frame", "token"):
            raise ValueError(f"access must be 'frame' or 'token' (got {access!r})")
        self.access = access
        self.check_finite = check_finite
        if access == "token":
            prepared = False
        self.shape = shape
        self.device = torch.device(device or "cuda")
        dt = shape.torch_dtype
        self.phi = [p.to(self.device, dt).contiguous() for p in (phi_q, phi_k, phi_v)]
        st = (shape.B, shape.H, shape.D, shape.D)
        self._S = [torch.zeros(st, dtype=torch.float32, device=self.device),
                   torch.zeros(st, dtype=torch.float32, device=self.device)]
        self._cur = 0
        ops = ((arl2.OP_TOKEN_LEVEL,) if access == "token" else
               (arl2.OP_READ, arl2.OP_READ_PREPARED, arl2.OP_CLEAN_PASS,
                arl2.OP_CLEAN_PASS_PREPARED, arl2.OP_COMMIT))
        ws_bytes = max(arl2.workspace_bytes(shape, op) for op in ops)
        self.ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=self.device)
        self.fused_clean = fused_clean
        self.seq = PassSequencer(n_denoise)
        # Reads of a frame all see the same S_{N-1}, so Phi_q S is formed once
        # per frame (after each commit) and every read uses it.
        self.prepared = prepared
        if prepared:
            # double-buffered like the state: the clean pass reads one map and
            # writes the next frame's into the other
            self._M = [arl2.alloc_prepared(shape, self.device),
                       arl2.alloc_prepared(shape, self.device)]
            self._mcur = 0
            self._prepare()

    @property
    def M(self) -> torch.Tensor:
        """The prepared map of S_{N-1} that the current frame's reads use."""
        return self._M[self._mcur]

    def _prepare(self, stream=None):
        if self.prepared:
            arl2.read_prepare(self.shape, self.phi[0], self.S, self.M, stream)

    @property
    def S(self) -> torch.Tensor:
        """The state every pass of the current frame reads (S_{N-1})."""
        return self._S[self._cur]

    @property
    def frame(self) -> int:
        return self.seq.frame

    def reset(self):
        for s in self._S:
            s.zero_()
        self._cur = 0
        self.seq.restore(0)
        self._prepare()

    def new_output(self):
        s = self.shape
        return torch.empty((s.B, s.H, s.T, s.D), dtype=s.torch_dtype, device=self.device)

    def read(self, q, k, v, o=None, o_intra=None, o_inter=None, stream=None, beta=None):
        """Denoising read against S_{N-1}; never writes the state. Under
        token-level access the in-frame updates need the frame's beta."""
        if self.access == "token" and beta is None:
            raise ValueError("token-level reads need the frame's beta")
        self.seq.before_read()
        if self.check_finite:
            check_finite(q=q, k=k, v=v, beta=beta)
        o = self.new_output() if o is None else o
        if self.access == "token":
            arl2.token_read(self.shape, q, k, v, *self.phi, beta, self.S, o, o_intra, o_inter,
                            self.ws, stream)
        elif self.prepared:
            arl2.read_prepared(self.shape, q, k, v, self.M, o, o_intra, o_inter, self.ws, stream)
        else:
            arl2.read(self.shape, q, k, v, self.phi[0], self.S, o, o_intra, o_inter, self.ws,
                      stream)
        self.seq.after_read()
        return o

    def clean_pass(self, q, k, v, beta, alpha, o=None, o_intra=None, o_inter=None, stream=None):
        """Read against S_{N-1}, commit S_N into the other buffer, swap."""
        self.seq.before_clean_pass()
        if self.check_finite:
            check_finite(q=q, k=k, v=v, beta=beta, alpha=alpha)
        o = self.new_output() if o is None else o
        nxt = 1 - self._cur
        if self.access == "token":
            arl2.token_clean_pass(self.shape, q, k, v, *self.phi, beta, alpha, self._S[self._cur],
                                  self._S[nxt], o, o_intra, o_inter, self.ws, stream)
        elif self.prepared and self.fused_clean:
            # also forms the next frame's map, into the other map buffer
            arl2.clean_pass_prepared(self.shape, q, k, v, self.M, self.phi[1], self.phi[2], beta,
                                     alpha, self._S[self._cur], self._S[nxt], o, o_intra,
                                     o_inter, self.ws, stream, phi_q=self.phi[0],
                                     prepared_next=self._M[1 - self._mcur])
            self._mcur = 1 - self._mcur
            self._cur = nxt
            self.seq.after_clean_pass()
            return o
        elif self.prepared:
            arl2.read_prepared(self.shape, q, k, v, self.M, o, o_intra, o_inter, self.ws, stream)
            arl2.commit(self.shape, k, v, self.phi[1], self.phi[2], beta, alpha,
                        self._S[self._cur], self._S[nxt], self.ws, stream)
        else:
            arl2.clean_pass(self.shape, q, k, v, self.phi[0], self.phi[1], self.phi[2], beta,
                            alpha, self._S[self._cur], self._S[nxt], o, o_intra, o_inter, self.ws,
                            stream)
        self._cur = nxt
        self.seq.after_clean_pass()
        self._prepare(stream)
        return o

    def commit(self, k, v, beta, alpha, stream=None):
        """State write of the clean pass without its read."""
        self.seq.before_clean_pass()
        if self.check_finite:
            check_finite(k=k, v=v, beta=beta, alpha=alpha)
        nxt = 1 - self._cur
        if self.access == "token":
            # the end state depends on K, V and beta only: any query will do,
            # and the read's outputs are discarded
            arl2.token_clean_pass(self.shape, k, k, v, *self.phi, beta, alpha, self._S[self._cur],
                                  self._S[nxt], self.new_output(), None, None, self.ws, stream)
        else:
            arl2.commit(self.shape, k, v, self.phi[1], self.phi[2], beta, alpha,
                        self._S[self._cur], self._S[nxt], self.ws, stream)
        self._cur = nxt
        self.seq.after_clean_pass()
        self._prepare(stream)

    # checkpoint / resume: the whole cross-frame memory is S plus the frame index
    def state_dict(self) -> dict:
        return {"S": self.S.detach().clone(), "frame": self.frame}

    def load_state_dict(self, sd: dict):
        S = sd["S"]
        if tuple(S.shape) != tuple(self.S.shape) or S.dtype != torch.float32:
            raise ValueError("state shape or dtype mismatch")
        self._S[0].copy_(S)
        self._cur = 0
        self.seq.restore(int(sd["frame"]))
        self._prepare()
