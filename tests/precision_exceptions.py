"""Where the stated precision itself misses the element-wise tolerance.

The parity bar is |gpu - oracle| <= 2e-2 + 1e-2 |oracle| per element, the
oracle in fp64.  The kernels compute in a stated mixed precision (bf16
operands of every matrix product -- q_hat, P, dS -- fp32 accumulation, bf16
outputs).  tests/rounding_model.py models exactly that arithmetic on the CPU.
In the cases named here the model itself lands outside the bound on a few
elements, by the same amount as the GPU; those elements are the precision's,
not a fault.

For a named (case, tensor) the GPU must still:
  * lie within the stated tolerance of the model at every element (it computes
    the stated arithmetic);
  * lie within the stated tolerance of the oracle, widened at each element by
    the model's own distance from the oracle there;
  * miss the plain bound on at most the count given here, and only where the
    model misses too.
Every other (case, tensor) takes the plain element-wise bound.

dW_g (the value-embedding gate's weight gradient) is a sum of dz x over every
token, up to a few hundred in size with terms of both signs; its elements of
small size cannot meet 2e-2 + 1e-2 |oracle| in the stated precision.  It is
always checked the named way, with no count limit.

"""

# (test case id, tensor): (elements outside the plain bound, their largest
# excess over it as measured on the GPU; the model's matched it)
ELEMENTWISE_EXCEPTIONS = {
    # value-embedding gate, 4 query heads per key/value head, window 0 (P = 1):
    # dve = gate * the sum of 4 heads' dO, rounded
    ("B2T308H12Hkv3D128W0C32reuse", "dve"): (1, 2.50e-5),
    # dx = dz W_g over 3 key/value heads
    ("B2T308H12Hkv3D128W0C32reuse", "dx32"): (2, 2.65e-3),
    # head size 64, the first keys of the sequence: large dS q_hat terms that
    # the RMSNorm backward's projection mostly cancels
    ("B1T181H6Hkv2D64W184C32", "dk"): (2, 1.00e-2),
    # dx with the rotary embedding, window 0
    ("B2T114H12Hkv3D128W0ropeC40", "dx32"): (1, 3.24e-3),
    # dq of one query, rotary embedding, full causal, 1000 keys
    ("B9T1000H8Hkv4D128W-1ropeC0", "dq"): (1, 9.24e-3),
}

# tensors always checked the named way
REDUCTIONS = ("dgate_w",)


def allowed(case_id: str, tensor: str):
    """None: the plain bound.  An int: the named check with that many elements
    allowed outside the plain bound; -1 for a reduction (no count limit)."""
    if tensor in REDUCTIONS:
        return -1
    e = ELEMENTWISE_EXCEPTIONS.get((case_id, tensor))
    return None if e is None else e[0]
