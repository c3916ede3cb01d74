"""Architecture definitions: parser and literal interpreter -- TEST INFRASTRUCTURE
(part of the oracle).

The text format is the one Synsema's "Local inference and architectures" page
defines in its section "The format":
  * header lines ``arch <name>``, ``kind decoder`` and ``param <key> <value>``;
  * three sections in the order ``prologue``, ``block`` (run once per layer,
    ``{i}`` replaced by the layer index) and ``epilogue``;
  * statements ``dst = op(src, ...)`` (assign to a register) or
    ``op(dst, ...)`` (change a register in place); ``#`` starts a comment;
  * tensors are named as the GGUF file names them, and ``a | b`` means tensor
    a, or b when a is absent; ``x`` is the residual register that links the
    layers; shapes (head_count, head_count_kv, embedding_length, the sliding
    window) come from the file's metadata, ``param`` lines only add what the
    file does not say.

The page lists the operations by name.  What each computes here (the plainest
reading consistent with the qwen3 file printed on that page and the Qwen3
walkthrough's Steps 2-9):
  embed(T)               rows of T for the tokens
  rms_norm(s, W)         RMSNorm over the last axis with gain W, eps from
                         <arch>.attention.layer_norm_rms_epsilon
  matmul(s, W)           s @ W^T, W stored [out][in] as GGUF rows
  add_bias(d, B)         d += B
  norm_heads(d, W, n)    RMSNorm of each of n heads of width key_length, gain W
  rope(d, n)             rotary embedding of n heads at the tokens' positions
  attention(q, k, v)     append k and v to the layer's cache, then causal (or
                         sliding-window) grouped-query attention
  silu / gelu / gelu_tanh / relu (d)   in place
  mul(d, s), add(d, s)   elementwise, in place
  scale(d, c)            d *= c, c a number
  copy(s)                the value of s
  last(s)                the last position only (kept whole when the logits of
                         every position are asked for)
Window layers (readings): a file with <arch>.attention.sliding_window needs a
``param window_pattern P``; layer i attends over the whole prefix iff
i % P == P - 1, the others over keys p - window < j <= p with the rotary base
``param rope_freq_base_local`` (default: <arch>.rope.freq_base).

The interpreter executes the statements one by one in float64, on the same
numerical primitives as ``oracle.model`` (``oracle.ops``), so that each op is
exactly its definition above; nothing is fused or reordered.
"""
import re
from dataclasses import dataclass, field

import numpy as np

from . import blocks
from . import ops

F64 = np.float64

# op -> (number of arguments, needs a destination register, argument kinds)
# kinds: r = register, t = tensor, n = metadata name or number
OPS = {
    "embed": ("t", True),
    "rms_norm": ("rt", False),
    "matmul": ("rt", False),
    "add_bias": ("rt", False),
    "norm_heads": ("rtn", False),
    "rope": ("rn", False),
    "attention": ("rrr", True),
    "silu": ("r", False),
    "gelu": ("r", False),
    "gelu_tanh": ("r", False),
    "relu": ("r", False),
    "mul": ("rr", False),
    "add": ("rr", False),
    "scale": ("rn", False),
    "copy": ("r", True),
    "last": ("r", False),
}
SECTIONS = ("prologue", "block", "epilogue")
PARAMS = ("window_pattern", "rope_freq_base_local")


class ArchdefError(ValueError):
    pass


@dataclass
class Stmt:
    dst: str      # register written (the first argument for in-place forms)
    op: str
    args: list
    line: int
    inplace: bool


@dataclass
class ArchDef:
    arch: str = ""
    kind: str = ""
    params: dict = field(default_factory=dict)
    sections: dict = field(default_factory=lambda: {s: [] for s in SECTIONS})


_STMT = re.compile(r"^(?:([A-Za-z_]\w*)\s*=\s*)?([A-Za-z_]\w*)\s*\((.*)\)$")
_REG = re.compile(r"^[A-Za-z_]\w*$")


def parse(text, name=None):
    """Parse a definition.  ``name`` (the file's base name), if given, must equal
    the declared architecture."""
    d = ArchDef()
    section = None
    seen = []
    for ln, raw in enumerate(text.splitlines(), 1):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        words = line.split()
        if line in SECTIONS:
            if line in seen:
                raise ArchdefError(f"line {ln}: section {line} twice")
            if seen and SECTIONS.index(line) < SECTIONS.index(seen[-1]):
                raise ArchdefError(f"line {ln}: section {line} out of order")
            seen.append(line)
            section = line
            continue
        if section is None:
            if words[0] == "arch" and len(words) == 2:
                d.arch = words[1]
            elif words[0] == "kind" and len(words) == 2:
                d.kind = words[1]
            elif words[0] == "param" and len(words) == 3:
                if words[1] not in PARAMS:
                    raise ArchdefError(f"line {ln}: unknown param {words[1]}")
                d.params[words[1]] = words[2]
            else:
                raise ArchdefError(f"line {ln}: expected arch, kind or param before the sections")
            continue
        m = _STMT.match(line)
        if not m:
            raise ArchdefError(f"line {ln}: not a statement")
        dst, op, argtext = m.group(1), m.group(2), m.group(3)
        if op not in OPS:
            raise ArchdefError(f"line {ln}: unknown operation {op}")
        args = [a.strip() for a in argtext.split(",")] if argtext.strip() else []
        kinds, needs_dst = OPS[op]
        if len(args) != len(kinds):
            raise ArchdefError(f"line {ln}: {op} takes {len(kinds)} arguments")
        for a, k in zip(args, kinds):
            if k == "r" and not _REG.match(a):
                raise ArchdefError(f"line {ln}: {a!r} is not a register")
            if k == "t" and not all(_tensor_name_ok(x) for x in _alternatives(a)):
                raise ArchdefError(f"line {ln}: {a!r} is not a tensor name")
        if needs_dst and dst is None:
            raise ArchdefError(f"line {ln}: {op} needs a destination (dst = {op}(...))")
        inplace = dst is None
        if inplace:
            dst = args[0]
        d.sections[section].append(Stmt(dst, op, args, ln, inplace))
    if not d.arch:
        raise ArchdefError("no arch line")
    if d.kind != "decoder":
        raise ArchdefError(f"kind must be decoder, got {d.kind!r}")
    if name is not None and name != d.arch:
        raise ArchdefError(f"the file {name}.archdef declares arch {d.arch}")
    if "block" not in seen:
        raise ArchdefError("no block section")
    return d


def _alternatives(a):
    return [x.strip() for x in a.split("|")]


def _tensor_name_ok(s):
    return bool(s) and re.match(r"^[A-Za-z0-9_.{}]+$", s) is not None and "." in s


class Interpreter:
    """Run a definition over a GGUF file's tensors, statement by statement.

    ``gguf`` is an ``oracle.gguf.GGUF`` (or anything with ``metadata`` and
    ``tensors``)."""

    def __init__(self, adef, gguf, max_ctx, n_seqs=1):
        self.d = adef
        self.md = gguf.metadata
        self.t = gguf.tensors
        a = adef.arch
        if self.md.get("general.architecture") != a:
            raise ArchdefError(f"the file is {self.md.get('general.architecture')!r}, the definition {a!r}")
        g = lambda k, dflt=None: self.md.get(f"{a}.{k}", dflt)  # noqa: E731
        self.n_layer = int(g("block_count"))
        self.hidden = int(g("embedding_length"))
        self.n_head = int(g("attention.head_count"))
        self.n_head_kv = int(g("attention.head_count_kv"))
        self.hd = int(g("attention.key_length", self.hidden // self.n_head))
        self.eps = float(g("attention.layer_norm_rms_epsilon"))
        self.theta = float(g("rope.freq_base", 10000.0))
        self.window = int(g("attention.sliding_window", 0))
        if self.window > 0 and "window_pattern" not in adef.params:
            raise ArchdefError("the file has a sliding window but the definition no window_pattern")
        self.pattern = int(adef.params.get("window_pattern", 0))
        self.theta_local = float(adef.params.get("rope_freq_base_local", self.theta))
        self.inv_g = ops.rope_inv_freq(self.theta, self.hd)
        self.inv_l = ops.rope_inv_freq(self.theta_local, self.hd)
        self.max_ctx = int(max_ctx)
        self.n_seqs = int(n_seqs)
        self.kv = [[None] * self.n_layer for _ in range(self.n_seqs)]
        self.kv_len = [0] * self.n_seqs
        self._w = {}

    # ------------------------------------------------------------ tensors
    def tensor(self, arg, layer):
        """Decoded tensor for an argument (``{i}`` substituted, first present alternative)."""
        for name in _alternatives(arg):
            name = name.replace("{i}", str(layer))
            if name in self.t:
                if name not in self._w:
                    t = self.t[name]
                    if t.data is None:
                        raise ArchdefError(f"tensor {name}: type {t.type} not readable")
                    w = blocks.dequant(t.type, t.data, t.rows, t.cols).astype(F64)
                    if len(t.ne) == 1:
                        w = w.reshape(-1)
                    self._w[name] = w
                return self._w[name]
        raise ArchdefError(f"tensor {arg.replace('{i}', str(layer))} is not in the file")

    def embed_rows(self, arg, tokens):
        for name in _alternatives(arg):
            if name in self.t:
                t = self.t[name]
                row_bytes = t.data.size // t.rows
                rows = t.data.reshape(t.rows, row_bytes)[np.asarray(tokens, dtype=np.int64)]
                return blocks.dequant(t.type, rows.reshape(-1), len(tokens), t.cols).astype(F64)
        raise ArchdefError(f"tensor {arg} is not in the file")

    def number(self, arg):
        if arg in ("head_count", "head_count_kv"):
            return self.n_head if arg == "head_count" else self.n_head_kv
        key = f"{self.d.arch}.{arg}"
        if key in self.md:
            return self.md[key]
        try:
            return float(arg)
        except ValueError:
            raise ArchdefError(f"{arg!r} is neither a number nor a metadata key") from None

    def is_global(self, layer):
        return self.window <= 0 or layer % self.pattern == self.pattern - 1

    # ------------------------------------------------------------ execution
    def _heads(self, x, n):
        T = x.shape[0]
        if x.shape[1] != n * self.hd:
            raise ArchdefError(f"register of width {x.shape[1]} is not {n} heads of {self.hd}")
        return x.reshape(T, n, self.hd).transpose(1, 0, 2)

    def _unheads(self, x):
        n, T, hd = x.shape
        return x.transpose(1, 0, 2).reshape(T, n * hd)

    def run(self, section, regs, layer, ctx):
        for s in self.d.sections[section]:
            try:
                self.step(s, regs, layer, ctx)
            except KeyError as e:
                raise ArchdefError(f"line {s.line}: register {e.args[0]} has no value") from None

    def step(self, s, regs, layer, ctx):
        op, a = s.op, s.args
        if op == "embed":
            v = self.embed_rows(a[0], ctx["tokens"])
        elif op == "rms_norm":
            v = ops.rmsnorm(regs[a[0]], self.tensor(a[1], layer), self.eps)
        elif op == "matmul":
            w = self.tensor(a[1], layer)
            if regs[a[0]].shape[1] != w.shape[1]:
                raise ArchdefError(f"line {s.line}: matmul of width {regs[a[0]].shape[1]} by {w.shape}")
            v = regs[a[0]] @ w.T
        elif op == "add_bias":
            v = regs[a[0]] + self.tensor(a[1], layer)
        elif op == "norm_heads":
            n = int(self.number(a[2]))
            v = self._unheads(ops.rmsnorm(self._heads(regs[a[0]], n), self.tensor(a[1], layer), self.eps))
        elif op == "rope":
            n = int(self.number(a[1]))
            inv = self.inv_g if self.is_global(layer) else self.inv_l
            ang = ops.rope_angles(ctx["pos"], inv)
            v = self._unheads(ops.apply_rope(self._heads(regs[a[0]], n), ang))
        elif op == "attention":
            v = self.attention(regs[a[0]], regs[a[1]], regs[a[2]], layer, ctx)
        elif op in ("silu", "gelu_tanh"):
            v = ops.ACTS[op](regs[a[0]])
        elif op == "gelu":
            v = ops.gelu_erf(regs[a[0]])
        elif op == "relu":
            v = np.maximum(regs[a[0]], 0.0)
        elif op == "mul":
            v = regs[a[0]] * regs[a[1]]
        elif op == "add":
            v = regs[a[0]] + regs[a[1]]
        elif op == "scale":
            v = regs[a[0]] * float(self.number(a[1]))
        elif op == "copy":
            v = regs[a[0]].copy()
        elif op == "last":
            v = regs[a[0]] if ctx["all_logits"] else regs[a[0]][-1:]
        else:  # pragma: no cover - parse() rejects unknown ops
            raise ArchdefError(f"line {s.line}: {op}")
        regs[s.dst] = v

    def attention(self, q, k, v, layer, ctx):
        seq, p0, pos = ctx["seq"], ctx["p0"], ctx["pos"]
        T = q.shape[0]
        if self.kv[seq][layer] is None:
            shape = (self.n_head_kv, self.max_ctx, self.hd)
            self.kv[seq][layer] = (np.zeros(shape, F64), np.zeros(shape, F64))
        K, V = self.kv[seq][layer]
        K[:, p0:p0 + T] = self._heads(k, self.n_head_kv)
        V[:, p0:p0 + T] = self._heads(v, self.n_head_kv)
        win = 0 if self.is_global(layer) else self.window
        o = ops.attention(self._heads(q, self.n_head), K[:, :p0 + T], V[:, :p0 + T], pos, win)
        return self._unheads(o)

    def forward(self, seq, tokens, all_logits=False):
        """Append ``tokens`` to sequence ``seq``: the epilogue's ``logits``
        register ([1][vocab], or [T][vocab] with all_logits)."""
        tokens = np.asarray(tokens, dtype=np.int64)
        T = len(tokens)
        p0 = self.kv_len[seq]
        if p0 + T > self.max_ctx:
            raise ValueError("context overflow")
        ctx = dict(seq=seq, p0=p0, pos=np.arange(p0, p0 + T), tokens=tokens, all_logits=all_logits)
        regs = {}
        self.run("prologue", regs, -1, ctx)
        for layer in range(self.n_layer):
            self.run("block", regs, layer, ctx)
        self.run("epilogue", regs, -1, ctx)
        self.kv_len[seq] = p0 + T
        if "logits" not in regs:
            raise ArchdefError("the epilogue does not assign logits")
        return regs["logits"]

    def decode(self, tokens):
        """One step for sequences 0..len(tokens)-1, one token each: logits [B][V]."""
        return np.concatenate([self.forward(s, [int(t)]) for s, t in enumerate(tokens)], axis=0)

    def reset(self, seq=-1):
        seqs = range(self.n_seqs) if seq < 0 else [seq]
        for s in seqs:
            self.kv_len[s] = 0
            self.kv[s] = [None] * self.n_layer


def config_from(adef, gguf):
    """The shape a definition and a file give (the keys of the synthetic
    configs), for comparing with the GPU library's view of the same file."""
    it = Interpreter(adef, gguf, max_ctx=1)
    return dict(n_layer=it.n_layer, hidden=it.hidden, n_head=it.n_head, n_head_kv=it.n_head_kv,
                head_dim=it.hd, vocab=gguf.tensors["token_embd.weight"].rows,
                ffn=int(gguf.metadata[f"{adef.arch}.feed_forward_length"]), rms_eps=it.eps,
                rope_theta=it.theta, rope_theta_local=it.theta_local, window=it.window,
                window_period=it.pattern if it.window > 0 else 0)
