"""Mask predicates ``allowed(i, j)`` written directly from the mask definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

These predicates are the oracle's notion of which (query i, key j) pairs are
admissible.  They are written from the text that defines each mask, never from
the HIP library's mask descriptor, so that the descriptor can be checked
against them bit for bit.

Teacher-forcing (TF) packed sequence, from "Causal-rCM ..." Section 3
(continuous-time consistency: tangents are computed through the TF-masked
packed forward; the clean context is fixed and only the noisy branch follows
the teacher) and Appendix B (packed clean-context and noisy-target tokens under
a TF mask), and "Causal Forcing ..." Section 2 (teacher forcing concatenates
clean and noisy videos with a causal attention mask):

* the sequence is ``[clean tokens | noisy tokens]``, each stream holding
  ``n_frames * tokens_per_frame`` tokens (clean first: the order is not stated
  on the pages; clean-first is the reading taken here);
* a *unit* is one frame (frame-wise) or ``frames_per_chunk`` consecutive frames
  (chunk-wise);
* a clean token of unit u sees every clean token of units u' <= u;
* a noisy token of unit u sees the clean tokens of units u' < u and the noisy
  tokens of its own unit u (bidirectional inside the unit), nothing else.

Each predicate object has ``n_q``, ``n_k`` and ``__call__(rows) -> bool
ndarray [len(rows), n_k]``.
"""

import numpy as np


class _Predicate:
    n_q: int
    n_k: int

    def __call__(self, rows):  # pragma: no cover - interface
        raise NotImplementedError

    def matrix(self):
        """Full [n_q, n_k] boolean matrix; for small masks only."""
        return self(np.arange(self.n_q))


class tf_allowed(_Predicate):
    """Teacher-forcing mask over the packed [clean | noisy] sequence.

    ``n_frames`` frames per stream, ``tokens_per_frame`` tokens per frame,
    ``frames_per_chunk`` frames per unit (1 = frame-wise).
    """

    def __init__(self, n_frames, tokens_per_frame, frames_per_chunk=1):
        if n_frames <= 0 or tokens_per_frame <= 0 or frames_per_chunk <= 0:
            raise ValueError("TF mask sizes must be positive")
        if n_frames % frames_per_chunk:
            raise ValueError("n_frames must be a multiple of frames_per_chunk")
        self.n_frames = n_frames
        self.tokens_per_frame = tokens_per_frame
        self.frames_per_chunk = frames_per_chunk
        self.n_clean = n_frames * tokens_per_frame
        self.unit_tokens = tokens_per_frame * frames_per_chunk
        self.n_q = self.n_k = 2 * self.n_clean

    def stream_and_unit(self, t):
        """(is_noisy, unit index) of token positions ``t``."""
        t = np.asarray(t, dtype=np.int64)
        is_noisy = t >= self.n_clean
        unit = (t % self.n_clean) // self.unit_tokens
        return is_noisy, unit

    def __call__(self, rows):
        q_noisy, q_unit = self.stream_and_unit(rows)
        k_noisy, k_unit = self.stream_and_unit(np.arange(self.n_k))
        qn, qu = q_noisy[:, None], q_unit[:, None]
        kn, ku = k_noisy[None, :], k_unit[None, :]
        clean_row = ~qn & ~kn & (ku <= qu)
        noisy_row_clean_key = qn & ~kn & (ku < qu)
        noisy_row_noisy_key = qn & kn & (ku == qu)
        return clean_row | noisy_row_clean_key | noisy_row_noisy_key


class dense_allowed(_Predicate):
    """Every query sees every key (plain attention)."""

    def __init__(self, n_q, n_k):
        self.n_q, self.n_k = n_q, n_k

    def __call__(self, rows):
        return np.ones((len(rows), self.n_k), dtype=bool)


class rects_allowed(_Predicate):
    """Union of query-key rectangles ("Causal-rCM ..." Appendix B: custom masks
    are query groups, each with its admissible key ranges).

    ``rects`` is a list of ``(q_begin, q_end, k_begin, k_end)`` half-open
    rectangles; a pair is admissible when it lies in at least one of them.
    """

    def __init__(self, n_q, n_k, rects):
        self.n_q, self.n_k = n_q, n_k
        self.rects = [tuple(int(x) for x in r) for r in rects]

    def __call__(self, rows):
        rows = np.asarray(rows, dtype=np.int64)
        keys = np.arange(self.n_k)
        out = np.zeros((len(rows), self.n_k), dtype=bool)
        for qb, qe, kb, ke in self.rects:
            rsel = (rows >= qb) & (rows < qe)
            ksel = (keys >= kb) & (keys < ke)
            out |= rsel[:, None] & ksel[None, :]
        return out


class block_causal_allowed(_Predicate):
    """Block-causal mask over a single stream of ``n_units`` units of
    ``unit_tokens`` tokens: a token of unit u sees units u' <= u.  This is the
    diffusion-forcing layout of "Causal Forcing ..." Section 2 (the noisy frame
    attends directly to the noisy prefix; no clean copy)."""

    def __init__(self, n_units, unit_tokens):
        self.n_units, self.unit_tokens = n_units, unit_tokens
        self.n_q = self.n_k = n_units * unit_tokens

    def __call__(self, rows):
        qu = np.asarray(rows, dtype=np.int64) // self.unit_tokens
        ku = np.arange(self.n_k) // self.unit_tokens
        return ku[None, :] <= qu[:, None]
