"""Arbitrary-precision brute force of masked softmax attention, for tiny inputs.

Pure Python loops over decimal.Decimal numbers (60 significant digits by
default), with no max shift: w_j = exp(s_j) directly.  Float inputs convert to
Decimal exactly, so the only rounding is decimal's, far below fp64's.  Used as
an independent pin of attention.py on tiny shapes (Nq, Nk, D of a few)."""
from decimal import Decimal, localcontext


def brute_attention(q, k, v, visible, scale, digits=60):
    """q [Nq][D], k [Nk][D], v [Nk][Dv] nested sequences of floats -> (o, lse) as floats."""
    with localcontext() as ctx:
        ctx.prec = digits
        sc = Decimal(float(scale))
        outs, lses = [], []
        for i, qi in enumerate(q):
            ws, vs = [], []
            for j, kj in enumerate(k):
                if not visible[i][j]:
                    continue
                s = sc * sum(Decimal(float(a)) * Decimal(float(b)) for a, b in zip(qi, kj))
                ws.append(s.exp())
                vs.append([Decimal(float(x)) for x in v[j]])
            if not ws:
                raise ValueError("a query row sees no key")
            l = sum(ws)
            o = [sum(w * vj[d] for w, vj in zip(ws, vs)) / l for d in range(len(vs[0]))]
            outs.append([float(x) for x in o])
            lses.append(float(l.ln()))
        return outs, lses
