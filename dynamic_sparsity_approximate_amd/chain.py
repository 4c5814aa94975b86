"""Chains of approximate matvecs on one stream.

The Effort method is applied per weight matrix with a per-call effort (Show HN
thread "Speeding up LLM inference 2x times (possibly)": effort is a real-time
knob; the author runs Mistral and Mixtral through it).  These classes only
sequence calls into libeffort and own the intermediate buffers; every step of
the arithmetic, the glue included (silu(h1) * h3, the gated expert sum), runs
in the library's kernels.  A caller that repeats a chain captures `enqueue`
into a HIP graph.
"""
from __future__ import annotations

import math

from . import binding as B

LAYER_ROLES = ("wq", "wk", "wv", "wo", "w1", "w3", "w2")


class EffortSchedule:
    """An effort for every matrix of a chain instead of one for all: the
    author's reply in the HN thread likens effort to an equalizer with a
    setting per layer, token and matrix rather than one knob; the reply to
    uhlo counts roughly 32 * 6 separate knobs per decode step.

    Keys are (layer, role) in a decode step (the head is (None, "head")) and
    (expert, role) in an expert block.  Lookup order: (unit, role), then
    (None, role) (a role's effort in every unit), then (unit, None) (a unit's
    effort for every role), then `default`.  Every effort must lie in (0, 1].
    """

    def __init__(self, default: float, table=None):
        self.default = float(default)
        self.table = {k: float(e) for k, e in dict(table or {}).items()}
        for k, e in [("default", self.default)] + list(self.table.items()):
            if not (0.0 < e <= 1.0):
                raise ValueError("effort %r for %r is outside (0, 1]" % (e, k))

    def __call__(self, unit, role) -> float:
        t = self.table
        for k in ((unit, role), (None, role), (unit, None)):
            if k in t:
                return t[k]
        return self.default

    @classmethod
    def from_array(cls, efforts, roles=LAYER_ROLES, head=None, default=None):
        """efforts[l][k] is the effort of roles[k] in layer l; `head` the output
        head's (default: the mean of the table)."""
        table = {}
        flat = []
        for l, row in enumerate(efforts):
            if len(row) != len(roles):
                raise ValueError("layer %d: %d efforts for %d roles" % (l, len(row), len(roles)))
            for r, e in zip(roles, row):
                table[(l, r)] = float(e)
                flat.append(float(e))
        mean = sum(flat) / len(flat) if flat else 1.0
        table[(None, "head")] = float(head) if head is not None else mean
        return cls(default if default is not None else mean, table)


def _effort_of(effort, unit, role) -> float:
    return float(effort(unit, role)) if callable(effort) else float(effort)


class DecodeStep:
    """All matvecs of one decode step of a decoder stack.

    `layers` is a list of dicts role -> EffortMatrix with the roles of
    LAYER_ROLES; `head` is the output projection.  Per layer l: wq, wk, wv, w1
    and w3 multiply the layer input x[l]; wo multiplies a[l] (attention, which
    produces wo's input, is outside this path); w2 multiplies silu(h1) * h3,
    formed from the approximate outputs h1 = x W1 and h3 = x W3.  The head
    multiplies `head_in`.  Inputs are device fp32 vectors supplied by the caller.
    With `grouped`, the matrices of a layer that share x go through one
    multi-matrix call each: (wq, wk, wv) and (w1, w3).
    """

    def __init__(self, layers, head, x, a, head_in, grouped: bool = False):
        import torch

        from .device import EffortGroup

        if len(layers) != len(x) or len(layers) != len(a):
            raise ValueError("one x and one a vector per layer")
        self.layers, self.head = layers, head
        self.x, self.a, self.head_in = x, a, head_in
        dev = head_in.device
        self.out = []
        for L in layers:
            o = {r: torch.empty(L[r].out_dim, dtype=torch.float32, device=dev) for r in LAYER_ROLES}
            o["g"] = torch.empty(L["w1"].out_dim, dtype=torch.float32, device=dev)
            self.out.append(o)
        self.logits = torch.empty(head.out_dim, dtype=torch.float32, device=dev)
        self.calls = 7 * len(layers) + 1
        self.groups = ([(EffortGroup([L["wq"], L["wk"], L["wv"]]), EffortGroup([L["w1"], L["w3"]]))
                        for L in layers] if grouped else None)

    def inputs_of(self, l: int) -> dict:
        """role -> the device vector that role's matvec multiplies in layer l."""
        o = self.out[l]
        return {"wq": self.x[l], "wk": self.x[l], "wv": self.x[l], "wo": self.a[l], "w1": self.x[l],
                "w3": self.x[l], "w2": o["g"]}

    def enqueue(self, effort, stream=None, side_streams=None, record=None):
        """Issue every call on `stream` (None: torch's current stream).
        `effort` is one effort for every matrix or an EffortSchedule (per
        layer and role; the head is (None, "head")).  With `side_streams`
        (torch streams), the six matvecs of a layer that do not depend on each
        other run on separate streams (parallel branches when captured into a
        graph); w2 and the next layer wait for them.  With `record` (a
        Recorder), every matvec records its parity outputs under (layer,
        role), the head under (None, "head")."""
        import torch

        main = stream if stream is not None else torch.cuda.current_stream()
        rk = (lambda key: None) if record is None else (lambda key: (record, key))  # noqa: E731
        for l, L in enumerate(self.layers):
            o, ins = self.out[l], self.inputs_of(l)
            roles = ("wq", "wk", "wv", "wo", "w1", "w3")
            e = {r: _effort_of(effort, l, r) for r in LAYER_ROLES}
            if self.groups:
                qkv, gu = self.groups[l]
                side = list(side_streams[:2]) if side_streams else []
                s_qkv = side[0] if side else main
                s_o = side[-1] if side else main
                for ss in side:
                    ss.wait_stream(main)
                qkv.matvec(self.x[l], [e["wq"], e["wk"], e["wv"]], [o["wq"], o["wk"], o["wv"]], s_qkv,
                           record=None if record is None else
                           (record, [(l, "wq"), (l, "wk"), (l, "wv")]))
                L["wo"].matvec(ins["wo"], e["wo"], o["wo"], s_o, record=rk((l, "wo")))
                gu.matvec(self.x[l], [e["w1"], e["w3"]], [o["w1"], o["w3"]], main,
                          record=None if record is None else (record, [(l, "w1"), (l, "w3")]))
                for ss in side:
                    main.wait_stream(ss)
            elif side_streams:
                for k, r in enumerate(roles):
                    ss = side_streams[k % len(side_streams)]
                    ss.wait_stream(main)
                    L[r].matvec(ins[r], e[r], o[r], ss, record=rk((l, r)))
                for ss in side_streams[:len(roles)]:
                    main.wait_stream(ss)
            else:
                for r in roles:
                    L[r].matvec(ins[r], e[r], o[r], main, record=rk((l, r)))
            B.effort_silu_mul(o["w1"], o["w3"], L["w1"].out_dim, o["g"], main)
            L["w2"].matvec(o["g"], e["w2"], o["w2"], main, record=rk((l, "w2")))
        self.head.matvec(self.head_in, _effort_of(effort, None, "head"), self.logits, main,
                         record=rk((None, "head")))


class DenseDecodeStep:
    """The same chain with the dense fp16 GEMV (weights as device fp16 [in][out])."""

    def __init__(self, layers, head, x, a, head_in):
        import torch

        self.layers, self.head = layers, head
        self.x, self.a, self.head_in = x, a, head_in
        dev = head_in.device
        self.out = []
        for L in layers:
            o = {r: torch.empty(L[r].shape[1], dtype=torch.float32, device=dev) for r in LAYER_ROLES}
            o["g"] = torch.empty(L["w1"].shape[1], dtype=torch.float32, device=dev)
            self.out.append(o)
        self.logits = torch.empty(head.shape[1], dtype=torch.float32, device=dev)

    def enqueue(self, stream=None, side_streams=None):
        import torch

        main = stream if stream is not None else torch.cuda.current_stream()
        roles = ("wq", "wk", "wv", "wo", "w1", "w3")
        for l, L in enumerate(self.layers):
            o = self.out[l]
            ins = {"wq": self.x[l], "wk": self.x[l], "wv": self.x[l], "wo": self.a[l],
                   "w1": self.x[l], "w3": self.x[l]}
            for k, r in enumerate(roles):
                ss = side_streams[k % len(side_streams)] if side_streams else main
                if ss is not main:
                    ss.wait_stream(main)
                m, n = L[r].shape
                B.dense_gemv(L[r], ins[r], m, n, o[r], ss)
            if side_streams:
                for ss in side_streams[:len(roles)]:
                    main.wait_stream(ss)
            B.effort_silu_mul(o["w1"], o["w3"], L["w1"].shape[1], o["g"], main)
            m, n = L["w2"].shape
            B.dense_gemv(L["w2"], o["g"], m, n, o["w2"], main)
        m, n = self.head.shape
        B.dense_gemv(self.head, self.head_in, m, n, self.logits, main)


def route_top2(logits):
    """Top-2 experts of a router's logits (ties go to the lower index) and their
    gates, the softmax over the two chosen logits (computed in double, returned
    as fp32 values)."""
    vals = [float(x) for x in logits]
    order = sorted(range(len(vals)), key=lambda e: (-vals[e], e))
    e0, e1 = order[0], order[1]
    z = math.exp(vals[e1] - vals[e0])
    g0 = 1.0 / (1.0 + z)
    g1 = z / (1.0 + z)
    return e0, e1, float(g0), float(g1)


class MoEFFN:
    """A mixture-of-experts feed-forward block: expert e is (w1, w3, w2) as
    EffortMatrix, y = g0 * FFN_e0(x) + g1 * FFN_e1(x) with FFN(x) =
    (silu(x W1) * x W3) W2.  Only the two routed experts' layouts are read.
    With `grouped`, the four matrices that multiply x (w1 and w3 of both
    routed experts) go through one multi-matrix call, one gate call covers
    both experts and the two w2 go through another multi-matrix call (side
    streams are then not used)."""

    def __init__(self, experts, device, grouped: bool = False):
        import torch

        self.experts = experts  # entries that are never routed to may be None
        first = next(e for e in experts if e is not None)
        d_in, d_hid = first[0].in_dim, first[0].out_dim
        self.d_in, self.d_hid = d_in, d_hid
        mk = lambda n: torch.empty(n, dtype=torch.float32, device=device)  # noqa: E731
        # both experts' hidden vectors side by side, so that one gate call
        # covers the pair
        self.h1_all, self.h3_all, self.g_all = mk(2 * d_hid), mk(2 * d_hid), mk(2 * d_hid)
        self.h1 = [self.h1_all[:d_hid], self.h1_all[d_hid:]]
        self.h3 = [self.h3_all[:d_hid], self.h3_all[d_hid:]]
        self.g = [self.g_all[:d_hid], self.g_all[d_hid:]]
        self.o = [mk(d_in), mk(d_in)]
        self.y = mk(d_in)
        self.grouped = grouped
        if grouped:  # one workspace serves every pair of experts (they share shapes)
            d4 = [first[0].desc, first[1].desc] * 2
            self.ws_bytes = B.effort_workspace_bytes_multi(d4)
            self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)
            d2 = [first[2].desc] * 2
            self.ws2_bytes = B.effort_workspace_bytes_multi(d2)
            self.ws2 = torch.zeros(self.ws2_bytes, dtype=torch.uint8, device=device)

    def enqueue(self, x, route, effort, stream=None, side_streams=None, record=None):
        """`effort` is one effort for all six matvecs or an EffortSchedule keyed
        by (expert, role), role in ("w1", "w3", "w2").  With `side_streams` (at
        least two torch streams), the two experts run on separate streams, and
        w1 / w3 of an expert on separate streams when there are four.  With
        `record` (a Recorder), every matvec records its parity outputs under
        (expert, role)."""
        import torch

        main = stream if stream is not None else torch.cuda.current_stream()
        e0, e1, g0, g1 = route
        ns = len(side_streams) if side_streams else 0
        ef = lambda e, r: _effort_of(effort, e, r)  # noqa: E731
        if self.grouped:
            mats = [self.experts[e0][0], self.experts[e0][1], self.experts[e1][0], self.experts[e1][1]]
            keys = [(e0, "w1"), (e0, "w3"), (e1, "w1"), (e1, "w3")]
            args = ([M.desc for M in mats], [M.layout for M in mats], x, [ef(*k) for k in keys],
                    [self.h1[0], self.h3[0], self.h1[1], self.h3[1]], self.ws, self.ws_bytes)
            if record is None:
                B.effort_matvec_multi(*args, stream=main)
            else:
                cutoff, K, rks, fp = record.multi(keys, [M.in_dim for M in mats])
                B.effort_matvec_multi_debug(*args, cutoff, K, rks, fp, stream=main)
            B.effort_silu_mul(self.h1_all, self.h3_all, 2 * self.d_hid, self.g_all, main)
            w2s = [self.experts[e0][2], self.experts[e1][2]]
            keys2 = [(e0, "w2"), (e1, "w2")]
            args2 = ([M.desc for M in w2s], [M.layout for M in w2s], self.g, [ef(*k) for k in keys2],
                     self.o, self.ws2, self.ws2_bytes)
            if record is None:
                B.effort_matvec_multi(*args2, stream=main)
            else:
                cutoff, K, rks, fp = record.multi(keys2, [M.in_dim for M in w2s])
                B.effort_matvec_multi_debug(*args2, cutoff, K, rks, fp, stream=main)
            B.effort_axpby(self.o[0], g0, self.o[1], g1, self.d_in, self.y, main)
            return self.y
        rk = (lambda key: None) if record is None else (lambda key: (record, key))  # noqa: E731
        for k, e in enumerate((e0, e1)):
            w1, w3, w2 = self.experts[e]
            s1 = side_streams[k % ns] if ns >= 2 else main
            s3 = side_streams[2 + k] if ns >= 4 else s1
            for ss in {s1, s3}:
                if ss is not main:
                    ss.wait_stream(main)
            w1.matvec(x, ef(e, "w1"), self.h1[k], s1, record=rk((e, "w1")))
            w3.matvec(x, ef(e, "w3"), self.h3[k], s3, record=rk((e, "w3")))
            if s3 is not s1:
                s1.wait_stream(s3)
            B.effort_silu_mul(self.h1[k], self.h3[k], self.d_hid, self.g[k], s1)
            w2.matvec(self.g[k], ef(e, "w2"), self.o[k], s1, record=rk((e, "w2")))
        if ns >= 2:
            for ss in side_streams[:2]:
                main.wait_stream(ss)
        B.effort_axpby(self.o[0], g0, self.o[1], g1, self.d_in, self.y, main)
        return self.y
