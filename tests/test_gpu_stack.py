"""GPU parity of the 65B layer stack: 80 layers x 7 linears (q, k, v, o 8192->8192;
gate, up 8192->22016; down 22016->8192), M = 2048 tokens, r = 64, with every NF4
weight resident in HBM at once (about 33 GB).  The forward runs over layers 0..79,
then the backward over 79..0, each linear on its own seeded inputs.

Three layers (the first, a middle and the last) are checked against the float64
oracle: the 8-bit block constants, group scales and mean in full and bit for bit;
the 4-bit codes of every block the sampled outputs read, bit for bit; Y on 96
sampled output columns and dX on two 64-column blocks (the last one included), for
every token row; T, dA and dB in full.
"""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_11_amd as Q
import workloads
from helpers import assert_close, host, host_u16, log, require_gpu
from oracle import linear, nf4

pytestmark = pytest.mark.gpu

CFG = workloads.CONFIGS[5]
SAMPLED = (0, 40, 79)
NCOLS = 96


def _sample(layer, slot):
    """Sampled output columns of Y and 64-column blocks of dX for one linear."""
    lin = CFG.linears[slot]
    rng = np.random.default_rng(7 * layer + slot)
    cols = np.sort(rng.choice(lin.d_out, NCOLS, replace=False))
    nkb = lin.d_in // 64
    kblk = np.array(sorted({int(rng.integers(0, nkb - 1)), nkb - 1}))
    return cols, kblk


def _blocks(lin, cols, kblk):
    """Block ids read by the sampled Y columns (whole weight rows) and dX columns."""
    nkb = lin.d_in // 64
    by = (cols[:, None] * nkb + np.arange(nkb)[None, :]).reshape(-1)
    bx = (np.arange(lin.d_out)[:, None] * nkb + kblk[None, :]).reshape(-1)
    return by, bx


@pytest.fixture(scope="module")
def stack():
    """Quantize all 560 weights, run the whole stack forward then backward, and keep
    host copies of what the sampled layers produced."""
    require_gpu()
    dev = torch.device("cuda", 0)
    lins = CFG.linears
    L = CFG.layers
    M, r = lins[0].M, lins[0].r
    ws = torch.empty(max(max(Q.qlora_quantize_workspace(l.d_out, l.d_in), Q.qlora_fwd_workspace(M, l.d_in, l.d_out, r),
                             Q.qlora_bwd_workspace(M, l.d_in, l.d_out, r)) for l in lins),
                     dtype=torch.uint8, device=dev)
    log("stack: drawing and quantizing", L * len(lins), "weights")
    wq, AB, X, dY, T = [], [], [], [], []
    for layer in range(L):
        row = []
        for j, lin in enumerate(lins):
            W = workloads.stack_tensor(layer, j, "W")
            row.append(Q.qlora_quantize_nf4(W, True, workspace=ws))
            del W
        wq.append(row)
        AB.append([(workloads.stack_tensor(layer, j, "A"), workloads.stack_tensor(layer, j, "B"))
                   for j in range(len(lins))])
        X.append({j: workloads.stack_tensor(layer, j, "X") for j in sorted(set(workloads.STACK_INPUT_SLOT))})
        dY.append([workloads.stack_tensor(layer, j, "dY") for j in range(len(lins))])
        T.append([torch.empty((M, r), dtype=torch.bfloat16, device=dev) for _ in lins])
    torch.cuda.synchronize()
    nf4_bytes = sum(w.nbytes() for row in wq for w in row)
    log(f"stack: {nf4_bytes / 1e9:.2f} GB of NF4 weight resident; "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")

    Y = [torch.empty((M, l.d_out), dtype=torch.bfloat16, device=dev) for l in lins]
    dX = [torch.empty((M, l.d_in), dtype=torch.bfloat16, device=dev) for l in lins]
    dA = [torch.empty((l.d_in, r), dtype=torch.float32, device=dev) for l in lins]
    dB = [torch.empty((r, l.d_out), dtype=torch.float32, device=dev) for l in lins]
    rec = {layer: [dict() for _ in lins] for layer in SAMPLED}
    for layer in range(L):
        for j, lin in enumerate(lins):
            x = X[layer][workloads.STACK_INPUT_SLOT[j]]
            A, B = AB[layer][j]
            Q.qlora_linear_fwd(x, wq[layer][j], A, B, lin.scale, Y=Y[j], T_save=T[layer][j], workspace=ws)
            if layer in SAMPLED:
                cols, _ = _sample(layer, j)
                rec[layer][j]["Y"] = host(Y[j][:, torch.from_numpy(cols).to(dev)].float())
    torch.cuda.synchronize()
    log("stack: forward over", L, "layers done")
    for layer in reversed(range(L)):
        for j, lin in enumerate(lins):
            x = X[layer][workloads.STACK_INPUT_SLOT[j]]
            A, B = AB[layer][j]
            Q.qlora_linear_bwd(dY[layer][j], x, T[layer][j], wq[layer][j], A, B, lin.scale, dX=dX[j], dA=dA[j],
                               dB=dB[j], workspace=ws)
            if layer in SAMPLED:
                _, kblk = _sample(layer, j)
                kcols = (kblk[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
                rec[layer][j]["dX"] = host(dX[j][:, torch.from_numpy(kcols).to(dev)].float())
                rec[layer][j]["dA"] = host(dA[j])
                rec[layer][j]["dB"] = host(dB[j])
    torch.cuda.synchronize()
    log("stack: backward over", L, "layers done")

    for layer in SAMPLED:
        for j, lin in enumerate(lins):
            w = wq[layer][j]
            cols, kblk = _sample(layer, j)
            by, bx = _blocks(lin, cols, kblk)
            sel = torch.from_numpy(np.concatenate([by, bx])).to(dev)
            d = rec[layer][j]
            d["codes"] = host(w.codes.view(-1, 32)[sel])
            d["c2"] = host(w.absmax)
            d["c1"] = host(w.c1)
            d["mu"] = host(w.mu)
            d["T"] = host(T[layer][j].float())
            d["X"] = host_u16(X[layer][workloads.STACK_INPUT_SLOT[j]])
            d["dY"] = host_u16(dY[layer][j])
            d["A"], d["B"] = host_u16(AB[layer][j][0]), host_u16(AB[layer][j][1])
    del wq, AB, X, dY, T, Y, dX, dA, dB, ws
    torch.cuda.empty_cache()
    return rec


@pytest.mark.parametrize("layer", SAMPLED)
def test_c5_stack_layer(stack, layer):
    for j in range(len(CFG.linears)):
        _check_linear(stack[layer][j], layer, j)


def _check_linear(d, layer, j):
    lin = CFG.linears[j]
    name = f"C5 layer {layer} {lin.name}"
    log(name, f"in={lin.d_in} out={lin.d_out}")
    W = host_u16(workloads.stack_tensor(layer, j, "W"))
    # block constants, in full and bit for bit
    absmax = nf4.blockwise_absmax(W)
    c2, c1, mu = nf4.double_quantize(absmax)
    assert np.array_equal(d["c2"], c2), f"{name}: 8-bit block constants differ"
    assert np.array_equal(d["c1"].view(np.uint32), np.asarray(c1, np.float32).view(np.uint32)), \
        f"{name}: group scales differ"
    assert d["mu"].view(np.uint32)[0] == np.float32(mu).view(np.uint32), f"{name}: mean differs"
    scales = nf4.block_scales_dq(c2, c1, mu)
    # codes of every block the sampled outputs read
    cols, kblk = _sample(layer, j)
    by, bx = _blocks(lin, cols, kblk)
    blocks = np.concatenate([by, bx])
    codes = nf4.codes_for_blocks(W, absmax, blocks)
    got = nf4.unpack_nibbles(d["codes"].reshape(-1), blocks.size * 64).reshape(blocks.size, 64)
    assert np.array_equal(got, codes), f"{name}: codes differ on {np.sum(np.any(got != codes, axis=1))} blocks"
    deq = nf4.dequantize_codes(codes.reshape(-1), scales[blocks]).reshape(blocks.size, 64)
    wrows = deq[:by.size].reshape(cols.size, lin.d_in)                      # W[cols][:]
    wcols = deq[by.size:].reshape(lin.d_out, kblk.size * 64)                # W[:][kcols]
    kcols = (kblk[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    # outputs: Y columns and T in full; dX columns; dA, dB in full
    y, t = linear.forward(d["X"], wrows, d["A"], d["B"][:, cols], lin.scale)
    assert_close(d["Y"], y, f"{name} Y cols")
    assert_close(d["T"], t, f"{name} T")
    dx = linear.backward_dx_rows(d["dY"], wcols, d["A"][kcols], d["B"], lin.scale, np.arange(lin.M))
    assert_close(d["dX"], dx, f"{name} dX cols")
    da, db = linear.adapter_grads(d["dY"], d["X"], d["A"], d["B"], lin.scale)
    assert_close(d["dA"], da, f"{name} dA")
    assert_close(d["dB"], db, f"{name} dB")
