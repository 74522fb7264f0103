"""Writes worked_examples.json: tiny SSD scans evaluated by hand.

Each case is small enough to unroll the recurrence of the nnterp guide,
"Mamba-2" page, opening section, by hand:

    h_t = exp(A d_t) h_{t-1} + d_t B_t x_t^T,   y_t = C_t^T h_t + D x_t,

with d_t = clamp(softplus(dt_t + dt_bias)) from section "The values".  The
expected numbers below are those hand derivations, evaluated with Python's
math module; no implementation of the scan is called.  Run from the repo
root: python tests/golden/make_worked_examples.py
"""
import json
import math
import os
import struct

E = math.exp
LN2 = math.log(2.0)


def f32(v):
    """The fp32 value the inputs are stored as (the scan reads fp32 inputs)."""
    return struct.unpack("f", struct.pack("f", v))[0]

cases = []

# 1. softplus off, A = -1, d = [0.5, 0.25], x = [1, 2], B = C = 1, D = 0, H0 = 0.
#    h1 = 0.5 * 1 * 1 = 0.5;  y1 = 0.5
#    h2 = e^{-0.25} * 0.5 + 0.25 * 1 * 2;  y2 = h2
h1 = 0.5
h2 = E(-0.25) * h1 + 0.25 * 2.0
cases.append(dict(
    name="two_tokens_no_softplus",
    derivation="h1 = d1 B1 x1 = 0.5; h2 = exp(A d2) h1 + d2 B2 x2 = e^-0.25 * 0.5 + 0.5",
    dims=dict(b=1, l=2, h=1, p=1, n=1, g=1),
    x=[1.0, 2.0], dt=[0.5, 0.25], A=[-1.0], B=[1.0, 1.0], C=[1.0, 1.0], D=[0.0],
    dt_bias=None, dt_softplus=False, dt_limit=[0.0, "inf"], init_state=None,
    y=[h1, h2], final=[h2]))

# 2. same with A = 0 (no decay): h2 = 0.5 + 0.5 = 1
cases.append(dict(
    name="two_tokens_no_decay",
    derivation="A = 0: h2 = h1 + d2 B2 x2 = 0.5 + 0.5 = 1",
    dims=dict(b=1, l=2, h=1, p=1, n=1, g=1),
    x=[1.0, 2.0], dt=[0.5, 0.25], A=[0.0], B=[1.0, 1.0], C=[1.0, 1.0], D=[0.0],
    dt_bias=None, dt_softplus=False, dt_limit=[0.0, "inf"], init_state=None,
    y=[0.5, 1.0], final=[1.0]))

# 3. same as 1 with D = 1: y gains x
cases.append(dict(
    name="two_tokens_skip",
    derivation="case 1 plus D x: y = [0.5 + 1, h2 + 2]",
    dims=dict(b=1, l=2, h=1, p=1, n=1, g=1),
    x=[1.0, 2.0], dt=[0.5, 0.25], A=[-1.0], B=[1.0, 1.0], C=[1.0, 1.0], D=[1.0],
    dt_bias=None, dt_softplus=False, dt_limit=[0.0, "inf"], init_state=None,
    y=[1.5, h2 + 2.0], final=[h2]))

# 4. softplus on: dt_raw = [0, z2] with z2 = fp32(ln(e - 1)) -> d = [ln 2, d2],
#    d2 = log(1 + e^z2) (= 1 up to the fp32 rounding of z2); A = -1; x = [1, 2];
#    B = [2, 1]; C = [1, 3]; D = 0.5.
#    h1 = ln2 * 2 * 1;  y1 = 1 * h1 + 0.5 * 1
#    h2 = e^{-d2} h1 + d2 * 1 * 2;  y2 = 3 h2 + 0.5 * 2
z2 = f32(math.log(math.e - 1.0))
d2 = math.log1p(math.exp(z2))
s1 = LN2 * 2.0
s2 = E(-d2) * s1 + d2 * 2.0
cases.append(dict(
    name="softplus_closed_form",
    derivation="softplus(0) = ln 2, softplus(z2) = log1p(e^z2) = d2 ~ 1; "
               "h1 = 2 ln 2; y1 = h1 + 0.5; h2 = e^-d2 h1 + 2 d2; y2 = 3 h2 + 1",
    dims=dict(b=1, l=2, h=1, p=1, n=1, g=1),
    x=[1.0, 2.0], dt=[0.0, z2], A=[-1.0], B=[2.0, 1.0],
    C=[1.0, 3.0], D=[0.5], dt_bias=None, dt_softplus=True, dt_limit=[0.0, "inf"],
    init_state=None, y=[s1 + 0.5, 3.0 * s2 + 1.0], final=[s2]))

# 5. clamp: dt_raw = [0, 0] with dt_bias = 1 -> softplus(1) = ln(1 + e) > 0.25,
#    dt_limit = (0, 0.25) -> d = [0.25, 0.25]; A = -2; x = [1, -1]; B = C = 1; D = 0.
c1 = 0.25
c2 = E(-2.0 * c1) * c1 + c1 * (-1.0)
cases.append(dict(
    name="time_step_limit",
    derivation="softplus(0 + 1) = 1.313 clamped to the limit c = 0.25; h1 = c; "
               "h2 = e^(-2c) c - c",
    dims=dict(b=1, l=2, h=1, p=1, n=1, g=1),
    x=[1.0, -1.0], dt=[0.0, 0.0], A=[-2.0], B=[1.0, 1.0], C=[1.0, 1.0], D=[0.0],
    dt_bias=[1.0], dt_softplus=True, dt_limit=[0.0, 0.25], init_state=None,
    y=[c1, c2], final=[c2]))

# 6. initial state: H0 = 3, A = -2, d = 0.5, x = B = C = 1, D = 0.
#    h1 = e^{-1} * 3 + 0.5
i1 = E(-1.0) * 3.0 + 0.5
cases.append(dict(
    name="initial_state",
    derivation="h1 = exp(A d) H0 + d B x = 3 e^-1 + 0.5",
    dims=dict(b=1, l=1, h=1, p=1, n=1, g=1),
    x=[1.0], dt=[0.5], A=[-2.0], B=[1.0], C=[1.0], D=[0.0],
    dt_bias=None, dt_softplus=False, dt_limit=[0.0, "inf"], init_state=[3.0],
    y=[i1], final=[i1]))

# 7. state layout [n, p] (state_dim first): n = 2, p = 3, one token, d = 1,
#    H0 = 0: h = B x^T = [[1, 10, 100], [2, 20, 200]];  C = (1, -1):
#    y = C^T h = [1 - 2, 10 - 20, 100 - 200].
cases.append(dict(
    name="state_layout_outer_product",
    derivation="h = d B x^T with B = (1, 2), x = (1, 10, 100): rows are state "
               "index, columns head_dim index; y_j = sum_i C_i h_ij",
    dims=dict(b=1, l=1, h=1, p=3, n=2, g=1),
    x=[1.0, 10.0, 100.0], dt=[1.0], A=[-1.0], B=[1.0, 2.0], C=[1.0, -1.0], D=[0.0],
    dt_bias=None, dt_softplus=False, dt_limit=[0.0, "inf"], init_state=None,
    y=[-1.0, -10.0, -100.0], final=[1.0, 10.0, 100.0, 2.0, 20.0, 200.0]))

# 8. dt = 0 skips a token exactly: tokens 1 and 3 write, token 2 has d = 0.
#    h1 = 0.5 * 1; h2 = h1 (exp(0) = 1, no write); h3 = e^{-0.5} h2 + 0.5 * 4
k1 = 0.5
k3 = E(-0.5) * k1 + 0.5 * 4.0
cases.append(dict(
    name="zero_time_step_skip",
    derivation="d2 = 0: exp(A * 0) = 1 and no write, so h2 = h1 = 0.5; "
               "h3 = e^-0.5 h2 + 2",
    dims=dict(b=1, l=3, h=1, p=1, n=1, g=1),
    x=[1.0, 7.0, 4.0], dt=[0.5, 0.0, 0.5], A=[-1.0], B=[1.0, 1.0, 1.0],
    C=[1.0, 1.0, 1.0], D=[0.0], dt_bias=None, dt_softplus=False,
    dt_limit=[0.0, "inf"], init_state=None, y=[k1, k1, k3], final=[k3]))

doc = dict(
    source="nnterp guide, 'Mamba-2' page: recurrence in the opening section; "
           "dt processing and the [b,h,n,p] state layout in 'The values'; dt = 0 "
           "as an exact skip in 'betas and decays are one argument'. The pages "
           "print no scan values: every number here is the hand unrolling "
           "recorded in 'derivation', evaluated with Python's math module.",
    cases=cases)

out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_examples.json")
with open(out, "w") as f:
    json.dump(doc, f, indent=1)
print("wrote", out)
