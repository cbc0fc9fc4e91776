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

here = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(here, "hand_examples.json"), "w") as f:
    json.dump({"source": "closed forms derived by hand; see make_hand_examples.py",
               "cases": cases}, f, indent=1)
print("wrote", len(cases), "cases")
