"""Writes hand_examples.json: two tiny forwards whose outputs follow by hand.

No implementation of the method is called; each expected value below is the
closed form derived in the comment beside it from the definitions on the pages:
routing = softmax over the router logits, top-k (CLIKA "MoE" page); linear =
x @ dequant(W).T (CLIKA "QLinearWoQ" page); dequant(q) = (q - 2^(bits-1)) * scale
with one scale per block_size elements along K (graiphic "QMoE" page, block_size,
expert_weight_bits); SwiGLU with alpha = 1, beta = 0 and no limit is silu(g) * u.

Run: python tests/golden/make_hand_examples.py
"""
import json
import math
import os
import struct


def sigmoid(v):
    return 1.0 / (1.0 + math.exp(-v))


cases = []

# Case 1 -- orientation of W (rows are outputs, K is contiguous), 8-bit, identity.
# x = e_0, W1[0][n][0] = (128 + 2n - 128) * 0.5 = n, so z = h = (0, 1, ..., 15).
# W2[0] = identity: W2[0][m][m] = (130 - 128) * 0.5 = 1, so y_m = m.
# logits (1, 0), k = 1, no renormalisation: w = e / (e + 1) = sigmoid(1).
# out_m = m * sigmoid(1).
cases.append(dict(
    name="orientation-8bit-identity",
    config=dict(H=16, I=16, E=2, k=1, bits=8, block_size=16, fusion=0, activation="identity",
                normalize=False),
    T=1,
    x=[[1.0] + [0.0] * 15],
    logits=[[1.0, 0.0]],
    w1_fill=128, w1_set=[[0, n, 0, 128 + 2 * n] for n in range(16)],
    s1=[0.5] * 32,
    w2_fill=128, w2_set=[[0, m, m, 130] for m in range(16)],
    s2_fill=0.5,
    expect=[[m * sigmoid(1.0) for m in range(16)]],
))

# Case 2 -- nibble order (element 2j+1 is the high nibble), concatenated gate/up, SwiGLU.
# x = e_1 selects the high nibble of byte 0 of every fc1 row.
# Expert 0: gate rows byte0 = 0x98 -> high nibble 9 -> g = (9 - 8) * 1 = 1;
#           up rows byte0 = 0xA8 -> high nibble 10 -> u = (10 - 8) * 1 = 2.
# h_i = silu(1) * 2 = 2 * sigmoid(1) for every i.
# fc2 expert 0: byte0 of each row = 0x89 -> element 0 (low nibble) 9 -> W2[m][0] = 0.5,
# every other element is the zero point, so y_m = 0.5 * h_0 = sigmoid(1).
# Expert 1 holds only zero points: its y is 0.
# logits (0.5, 0), k = 2, renormalised over both = the softmax: w_0 = sigmoid(0.5).
# out_m = sigmoid(0.5) * sigmoid(1).
cases.append(dict(
    name="nibble-order-4bit-swiglu-concat",
    config=dict(H=32, I=16, E=2, k=2, bits=4, block_size=16, fusion=2, activation="swiglu",
                normalize=True),
    T=1,
    x=[[0.0, 1.0] + [0.0] * 30],
    logits=[[0.5, 0.0]],
    w1_fill=0x88,
    w1_set=[[0, n, 0, 0x98] for n in range(16)] + [[0, 16 + n, 0, 0xA8] for n in range(16)],
    s1=[1.0] * (2 * 32 * 2),
    w2_fill=0x88, w2_set=[[0, m, 0, 0x89] for m in range(32)],
    s2_fill=0.5,
    expect=[[sigmoid(0.5) * sigmoid(1.0)] * 32],
))

# Sparse mixer routing (graiphic "QMoE" page, use_sparse_mixer; CLIKA "MoE" page,
# sparse_mixer_eps; the SparseMixer top-2 router as published for Phi-3.5-MoE): pick 1 is
# the largest logit m1, pick 2 the largest of the others m2 (ties: lower index). A pick
# keeps expert e unless (m - l_e) / max(|l_e|, m) > 2 eps (the second pick never keeps
# the first); its weight is exp(m - m) / sum over the kept experts of exp(l_e - m).
# The logits are stored as float32, so each closed form below uses the float32 values
# (f32() rounds a literal the way the stored logit is rounded).


def f32(v):
    return struct.unpack("<f", struct.pack("<f", v))[0]


mixer = []
eps = 0.01
# A: l = (2, 1.99, 0.5, -1). Pick 1 (expert 0, m = 2): expert 1 trails by 0.01/2 = 0.005
# <= 0.02 and is kept; 0.5 trails by 1.5/2 and -1 by 3/2: dropped. w1 = 1/(1 + e^(l1-l0)).
# Pick 2 (expert 1, m = 1.99): 0.5 trails by 1.49/1.99, -1 by 2.99/1.99: dropped; w2 = 1.
la = [f32(2.0), f32(1.99), f32(0.5), f32(-1.0)]
mixer.append(dict(name="keeps-a-near-tie", eps=eps, logits=[la],
                  ids=[[0, 1]], w=[[1.0 / (1.0 + math.exp(la[1] - la[0])), 1.0]]))
# B: negative logits (-1, -1.01, -1.015, -3). Pick 1 (m = -1, so max(|l|, m) = |l|):
# 0.01/1.01 and 0.015/1.015 are kept, 2/3 is dropped. w1 = 1/(1 + e^(l1-l0) + e^(l2-l0)).
# Pick 2 (expert 1, m = -1.01): expert 2 trails by 0.005/1.015 (kept), expert 3 by 1.99/3
# (dropped). w2 = 1/(1 + e^(l2-l1)).
lb = [f32(-1.0), f32(-1.01), f32(-1.015), f32(-3.0)]
mixer.append(dict(name="negative-logits", eps=eps, logits=[lb], ids=[[0, 1]],
                  w=[[1.0 / (1.0 + math.exp(lb[1] - lb[0]) + math.exp(lb[2] - lb[0])),
                      1.0 / (1.0 + math.exp(lb[2] - lb[1]))]]))
# C: ties (1, 1, 0, 1). Pick 1 takes expert 0; the other 1s trail by 0 (kept), the 0 by
# 1/1 (dropped): w1 = 1/3. Pick 2 takes expert 1 (the lowest of the remaining ties), keeps
# expert 3: w2 = 1/2.
mixer.append(dict(name="ties-to-lower-index", eps=eps, logits=[[1.0, 1.0, 0.0, 1.0]],
                  ids=[[0, 1]], w=[[1.0 / 3.0, 0.5]]))
# D: zero logits (0, 0, -0.5, 0). Pick 1 (m = 0): the other zeros give 0/0, which is not
# above the threshold, so they are kept; -0.5 trails by 0.5/0.5 = 1: dropped. w1 = 1/3.
# Pick 2 (expert 1, m = 0) keeps expert 3 the same way: w2 = 1/2.
mixer.append(dict(name="zero-over-zero-keeps", eps=eps, logits=[[0.0, 0.0, -0.5, 0.0]],
                  ids=[[0, 1]], w=[[1.0 / 3.0, 0.5]]))
# E: eps = 0.3 (threshold 0.6) on (4, 1, 3, 2): pick 1 (m = 4) keeps 3 (1/4) and 2
# (2/4), drops 1 (3/4): w1 = 1/(1 + e^-1 + e^-2). Pick 2 takes expert 2 (m = 3): expert 3
# trails by 1/3 (kept), expert 1 by 2/3 (dropped): w2 = 1/(1 + e^-1).
mixer.append(dict(name="wide-threshold", eps=0.3, logits=[[4.0, 1.0, 3.0, 2.0]],
                  ids=[[0, 2]],
                  w=[[1.0 / (1.0 + math.exp(-1.0) + math.exp(-2.0)), 1.0 / (1.0 + math.exp(-1.0))]]))

# F: the denominator is max(|l|, m), not |m|: l = (-1, -1.0204, -5, -6). Pick 1 (m = -1):
# expert 1 trails by 0.0204 / 1.0204 = 0.019992 <= 0.02 and is kept (0.0204 / |m| would
# drop it); experts 2 and 3 trail by 4/5 and 5/6: dropped. w1 = 1/(1 + e^(l1-l0)).
# Pick 2 (expert 1) drops experts 2 and 3 (3.98/5, 4.98/6): w2 = 1.
lf = [f32(-1.0), f32(-1.0204), f32(-5.0), f32(-6.0)]
mixer.append(dict(name="denominator-is-max-of-abs-and-pick", eps=eps, logits=[lf],
                  ids=[[0, 1]], w=[[1.0 / (1.0 + math.exp(lf[1] - lf[0])), 1.0]]))

here = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(here, "hand_examples.json"), "w") as f:
    json.dump({"source": "closed forms derived by hand; see make_hand_examples.py",
               "cases": cases, "mixer_cases": mixer}, f, indent=1)
print("wrote", len(cases), "forward cases and", len(mixer), "sparse mixer cases")
