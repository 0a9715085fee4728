"""Algorithmic HBM bytes of each decode-path launch (the traffic model).

Eager decoding moves the whole [B,H,dk,dv] state twice per token although a
token adds only O(dk + dv) numbers per head (gist.science summary, section
"Problema").  DeltaLog replaces the dense write of M-1 out of every M tokens
with compact appends and one amortised dense write (section "Modello di
Traffico").  These functions count the bytes each launch must move at
minimum -- every input, log entry and state element read or written once --
which is what "achieved GB/s" divides by.  The C library's
dl_predict_token_us / dl_choose_capacity implement the same model.

Per head, dk key and dv value channels, s = input element size (4 fp32, 2 bf16):
  base tile        4 dk dv
  token inputs     q|r, k: 2 dk s; v: dv s; beta 4 (delta rules); decay 4 (GDN) or 4 dk
  output           4 dv
  log entry        X: 4 dv (u, delta rules) or dv s (v, RWKV6); K: dk s; G: 4 or 4 dk
  RWKV6 bonus      4 dk per attention head, read once per launch (H rows)
An append at log length L reads the base, the token and L entries and writes
one entry and the output; the fused fold (L = C-1) also writes the base and
writes no entry; eager reads and writes the state.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Shape:
    op: str
    B: int
    H: int
    d: int         # key width dk (and the value width when dv is 0)
    in_bytes: int  # 4 (fp32) or 2 (bf16)
    dv: int = 0    # value width; 0 means dv = d

    @property
    def heads(self):
        return self.B * self.H

    @property
    def dk(self):
        return self.d

    @property
    def dvv(self):
        return self.dv or self.d

    def base(self):
        return 4 * self.dk * self.dvv

    def token_in(self):
        s = self.in_bytes
        b = (2 * self.dk + self.dvv) * s
        if self.op != "rwkv6":
            b += 4  # beta
        b += 4 if self.op == "gdn" else 4 * self.dk
        return b

    def out(self):
        return 4 * self.dvv

    def entry(self):
        s = self.in_bytes
        x = self.dvv * s if self.op == "rwkv6" else 4 * self.dvv
        g = 4 if self.op == "gdn" else 4 * self.dk
        return x + self.dk * s + g

    def shared(self):
        return 4 * self.dk * self.H if self.op == "rwkv6" else 0


def append_bytes(sh: Shape, L: int) -> int:
    """An append at log length L (the token becomes entry L)."""
    per = sh.base() + sh.token_in() + sh.out() + (L + 1) * sh.entry()
    return sh.heads * per + sh.shared()


def merge_bytes(sh: Shape, C: int) -> int:
    """The token that fills the log (L = C-1) fused with the fold into the base."""
    per = 2 * sh.base() + sh.token_in() + sh.out() + (C - 1) * sh.entry()
    return sh.heads * per + sh.shared()


def eager_bytes(sh: Shape) -> int:
    per = 2 * sh.base() + sh.token_in() + sh.out()
    return sh.heads * per + sh.shared()


def chunk_bytes(sh: Shape, L: int, K: int, fold: bool) -> int:
    """K tokens in one launch at log length L: one base read (and write when
    the chunk fills the log), K tokens in and out, L entries replayed, and the
    K new entries written unless they are folded."""
    per = sh.base() * (2 if fold else 1) + K * (sh.token_in() + sh.out()) + L * sh.entry()
    if not fold:
        per += K * sh.entry()
    return sh.heads * per + sh.shared()


def call_bytes(sh: Shape, L: int, K: int, C: int) -> int:
    """K tokens in one launch from log length L, folding whenever the log
    fills: one read of the base, one write per fold, every token in and out,
    the L old entries replayed, and the entries that remain in the log after
    the call (the tokens past its last fold) written."""
    per = sh.base()
    left, l = K, L
    while left > 0:
        k = min(left, C - l)
        fold = l + k == C
        per += k * (sh.token_in() + sh.out()) + l * sh.entry()
        per += sh.base() if fold else k * sh.entry()
        l = 0 if fold else l + k
        left -= k
    return sh.heads * per + sh.shared()


def multi_token_bytes(sh: Shape, C: int, K: int, ntokens: int, L: int = 0) -> int:
    """ntokens tokens decoded in calls of K from log length L."""
    total, left = 0, ntokens
    while left > 0:
        k = min(K, left)
        total += call_bytes(sh, L, k, C)
        L = (L + k) % C
        left -= k
    return total


def fold_bytes(sh: Shape, L: int) -> int:
    """A standalone fold (merge or materialise) of L entries."""
    return sh.heads * (2 * sh.base() + L * sh.entry())


def cycle_bytes(sh: Shape, C: int) -> int:
    """One merge cycle of C tokens: C-1 appends and the fused fold."""
    if C == 1:
        return merge_bytes(sh, 1)
    return sum(append_bytes(sh, L) for L in range(C - 1)) + merge_bytes(sh, C)


def per_token_bytes(sh: Shape, C: int) -> float:
    return cycle_bytes(sh, C) / C


def cycle_flops(sh: Shape, C: int) -> int:
    """Useful FLOPs of one cycle: the base mat-vecs (two for delta rules, one
    for RWKV6) every token, plus the rank-C fold and row scaling once."""
    mv = (4 if sh.op != "rwkv6" else 2) * sh.dk * sh.dvv
    fold = 2 * C * sh.dk * sh.dvv + sh.dk * sh.dvv
    return sh.heads * (C * mv + fold)
