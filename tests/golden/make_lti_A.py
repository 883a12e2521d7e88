"""Writes lti_A.json: closed-form values of the LTI diagonal.

[ZS] "OpenMythos 분석 …", §latent reasoning: A = exp(-exp(clamp(log_dt +
log_A, -20, 20))).  [RC] "OpenMythos", §해결책: the same A is the zero-order
hold exp(dt * A_c) of A_c = -exp(log_A) with dt = exp(log_dt).  Values are
evaluated here with Python's math module in double precision.
"""
import json
import math
import os

cases = []
for log_dt, log_A in [(0.0, [-30.0, -1.0, 0.0, 1.0, 30.0]), (-2.0, [0.5, -19.0, 25.0])]:
    exp = []
    for la in log_A:
        s = min(20.0, max(-20.0, log_dt + la))
        exp.append(math.exp(-math.exp(s)))
    cases.append(dict(log_dt=log_dt, log_A=log_A, expected=exp))
out = dict(source="closed form of the LTI diagonal with the [-20, 20] clamp", cases=cases)
json.dump(out, open(os.path.join(os.path.dirname(__file__), "lti_A.json"), "w"), indent=1)
