"""Host driver of one denoise step over a single request's canvas: the three library
calls in their order, on buffers fixed once.

A step ([P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM",
sections "샘플링 루프와 엔트로피 경계 디노이징" and "ModelState 인터페이스") is
  1. attention of the canvas over its committed prefix (dg_attn_mixed),
  2. the DiffusionSampler step on the step's logits (dg_sampler_step), which also
     records whether the block has converged,
  3. the self-conditioning average of the embeddings under the step's softmax
     (dg_selfcond_embed), which the next step's input side consumes.
Every argument struct is built once; a step only edits the request's step index and
seed and passes the structs to the library. Nothing here computes: the arithmetic is
in the kernels behind the calls.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import (DG_CONV_OR, DG_INIT_CANVAS, SamplerBuffers, prepare_attn, prepare_sampler, prepare_selfcond)

MASK64 = (1 << 64) - 1


class DenoiseStep:
    """The calls of one denoise step of one request.

    q, k, v, seqs, window, hq, hkv: the attention layer (one request's canvas over its
    prefix); logits: one or more [M, V] tensors, the step picks one by index (a loop
    driver that cycles through precomputed logits); embed [V, d]: the embedding table.
    selfcond_input: "probs", the sampler also writes block-scaled probabilities that
    self-conditioning reads; "logits", self-conditioning reads the logits with the
    sampler's row statistics (p = exp(l - row_max) / row_sum).
    """

    def __init__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seqs: Sequence, window: int, hq: int,
                 hkv: int, logits: List[torch.Tensor], embed: torch.Tensor, budget: float, stable_k: int,
                 tau: float, step_limit: int, combine: int = DG_CONV_OR, seed: int = 0,
                 selfcond_input: str = "probs"):
        dev = q.device
        M, V = logits[0].shape
        self.rows, self.vocab, self.seed = M, V, seed
        self.attn_out = torch.empty_like(q)
        self.lse = torch.empty(q.shape[0], hq, device=dev, dtype=torch.float32)
        probs = selfcond_input == "probs"
        if not probs and selfcond_input != "logits":
            raise ValueError(f"selfcond_input must be 'probs' or 'logits', not {selfcond_input!r}")
        self.bufs = SamplerBuffers(M, 1, dev, vocab=V if probs else 0, probs_dtype=logits[0].dtype if probs else None)
        self.sc_out = torch.empty(M, embed.shape[1], device=dev, dtype=embed.dtype)
        self.logits = logits
        self.attn = prepare_attn(q, k, v, self.attn_out, seqs, window, hq, hkv, lse=self.lse)
        kw = dict(stable_k=stable_k, tau=tau, step_limit=step_limit, combine=combine, probs=self.bufs.probs,
                  probs_scale=self.bufs.probs_scale)
        self.samp = [prepare_sampler(l, [(0, M, seed, 0)], V, self.bufs, budget, **kw) for l in logits]
        self.init = prepare_sampler(None, [(0, M, seed, 0)], V, self.bufs, budget, flags=DG_INIT_CANVAS,
                                    num_rows=M)
        if probs:  # one call: the probabilities buffer is the same whatever the logits
            sc = prepare_selfcond(self.bufs.probs, embed, self.sc_out, p_scale=self.bufs.probs_scale)
            self.selfcond = [sc] * len(logits)
        else:
            sc = prepare_selfcond(logits[0], embed, self.sc_out, row_max=self.bufs.row_max, row_sum=self.bufs.row_sum)
            self.selfcond = [sc] + [prepare_selfcond(l, embed, self.sc_out, row_max=self.bufs.row_max,
                                                     row_sum=self.bufs.row_sum, workspace=sc._keep[0])
                                    for l in logits[1:]]

    def start_block(self, seed: int, stream=None) -> None:
        """A new block: a random canvas and reset state (the sampler's init call)."""
        self.seed = seed & MASK64
        r = self.init.args._keep[0]
        r.step, r.seed = 0, self.seed
        self.init(stream)

    def enqueue(self, t: int, which: int, stream=None, converged_ptr: Optional[int] = None, flags: int = 0,
                events=None) -> None:
        """Enqueue step t of the current block on `stream`, with logits[which].
        converged_ptr: device-accessible int32 that receives the converged flag (None:
        the sampler buffers' own). flags: extra sampler flags (e.g. DG_ENTROPY_IN).
        events: None, or four events recorded before attention, after it, after the
        sampler and after self-conditioning."""
        samp = self.samp[which]
        r = samp.args._keep[0]
        r.step, r.seed = t, self.seed
        samp.args.flags = flags
        samp.args.converged = converged_ptr if converged_ptr is not None else self.bufs.converged.data_ptr()
        if events is not None:
            events[0].record(stream)
        self.attn(stream)
        if events is not None:
            events[1].record(stream)
        samp(stream)
        if events is not None:
            events[2].record(stream)
        self.selfcond[which](stream)
        if events is not None:
            events[3].record(stream)
