"""Chains of batch-1 products in one persistent launch (lowbit_chain_*).

Every stage of a chain must meet the oracle tolerance, and where its rows
are reduced in one K-slice it must reproduce a separate lowbit_gemv call
bit for bit (the same per-group arithmetic in the same order; longer rows
may be cut into different slices); a chain whose stage i reads stage i-1's
output as its activations must match the oracle applied stage by stage to
the GPU's own intermediate outputs, and must equal the separate calls on
those same intermediates."""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from ultra_bit_dit_amd import lowbit as lb

from helpers import SEED, assert_within, codes_for, silu_mul_tolerance, to_np

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make(fmt, N, K, tid):
    codes = codes_for(fmt, SEED, tid, N, K)
    scales = synth.group_scales(SEED, tid + 1, N, K // 128)
    pc, ps = lb.pack(fmt, dev(codes), dev(scales.view(np.int16)))
    return codes, scales, pc, ps


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("wait", [0, 1])
def test_chain_matches_separate_calls(fmt, wait):
    # (48, 20480): four K-slices per row group; the binary streaming kernel
    # gives each wave three row-blocks, so 100 and 3000 rows leave a last
    # wave with one and with two live row-blocks
    shapes = [(640, 1024), (100, 5120), (256, 17408), (5120, 5120), (48, 128), (3000, 2560),
              (48, 20480), (20480, 2560)]
    mats, xs, ys, refs = [], [], [], []
    for j, (N, K) in enumerate(shapes):
        codes, scales, pc, ps = make(fmt, N, K, tid=200 + 2 * j)
        mats.append((pc, ps))
        xh = synth.normal_bf16(SEED, 230 + j, 1, K)
        xs.append(dev(xh.view(np.int16)).view(torch.bfloat16)[0])
        ys.append(torch.full((N,), float("nan"), device="cuda"))
        refs.append(O.matmul(codes, scales, O.X_BF16, xh))
    stages = [(fmt, N, K, mats[j][0], mats[j][1], xs[j], ys[j], wait)
              for j, (N, K) in enumerate(shapes)]
    chain = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32)
    for rep in range(3):  # counters must be left at zero by every run
        for y in ys:
            y.fill_(float("nan"))
        chain.run()
        torch.cuda.synchronize()
        for j, (N, K) in enumerate(shapes):
            yref, absY = refs[j]
            assert_within(ys[j].cpu().numpy()[None], yref, absY, what=f"stage {j} run {rep}")
            if K <= 5120 and lb.workspace_bytes(fmt, 1, N, K, lb.BF16) == 256 << 10:
                # one K-slice in both kernels (the one-product call holds no
                # split-K partials: it was not split to fill the device): the
                # same arithmetic in the same order
                ref = lb.gemv(fmt, N, K, mats[j][0], mats[j][1], xs[j])
                torch.cuda.synchronize()
                assert torch.equal(ys[j], ref), f"stage {j} run {rep}"
    assert chain.failed_waits() == 0
    chain.close()


@pytest.mark.parametrize("fmt", [1, 2])
def test_chain_dependent_stages(fmt):
    """x of stage i is y of stage i-1 (fp32): each stage must wait for the
    whole previous product."""
    dims = [1024, 640, 5120, 384, 256, 20480, 1024]
    mats, codes, scales = [], [], []
    for j in range(len(dims) - 1):
        K, N = dims[j], dims[j + 1]
        c, s, pc, ps = make(fmt, N, K, tid=260 + 2 * j)
        mats.append((pc, ps))
        codes.append(c)
        scales.append(s)
    x0 = synth.normal_f32(SEED, 290, 1, dims[0])
    bufs = [dev(x0)[0]] + [torch.full((d,), float("nan"), device="cuda") for d in dims[1:]]
    stages = [(fmt, dims[j + 1], dims[j], mats[j][0], mats[j][1], bufs[j], bufs[j + 1], 1)
              for j in range(len(dims) - 1)]
    chain = lb.Chain(stages, x_dtype=lb.F32, y_dtype=lb.F32)
    for rep in range(3):
        for b in bufs[1:]:
            b.fill_(float("nan"))
        chain.run()
        torch.cuda.synchronize()
        outs = [b.cpu().numpy() for b in bufs]
        for j in range(len(dims) - 1):
            xin = outs[j][None].astype(np.float32)
            yref, absY = O.matmul(codes[j], scales[j], O.X_F32, xin)
            assert_within(outs[j + 1][None], yref, absY, what=f"stage {j} run {rep}")
            sep = lb.gemv(fmt, dims[j + 1], dims[j], mats[j][0], mats[j][1], bufs[j])
            torch.cuda.synchronize()
            if lb.workspace_bytes(fmt, 1, dims[j + 1], dims[j], lb.F32) == 256 << 10:
                # the one-product call runs one K-slice too: the same order
                assert torch.equal(sep, bufs[j + 1])
            else:  # it was split along K to fill the device: the bound instead
                assert_within(sep.cpu().numpy()[None], yref, absY, what=f"separate {j}")
    assert chain.failed_waits() == 0
    chain.close()


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_chain_waiting_second_items(fmt):
    """A waiting product with more work items than resident workgroups
    (19200 x 10240: 300 row groups x 2 K-slices = 600 items): the workgroups
    that run a second item of the same K-slice warm its codes and scales
    before their first wait.  Every output must still meet the oracle."""
    shapes = [(640, 1024), (19200, 10240)]
    mats, xs, ys, refs = [], [], [], []
    for j, (N, K) in enumerate(shapes):
        codes, scales, pc, ps = make(fmt, N, K, tid=320 + 2 * j)
        mats.append((pc, ps))
        xh = synth.normal_bf16(SEED, 340 + j, 1, K)
        xs.append(dev(xh.view(np.int16)).view(torch.bfloat16)[0])
        ys.append(torch.full((N,), float("nan"), device="cuda"))
        refs.append(O.matmul(codes, scales, O.X_BF16, xh))
    stages = [(fmt, N, K, mats[j][0], mats[j][1], xs[j], ys[j], 1) for j, (N, K) in enumerate(shapes)]
    chain = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32)
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        chain.run()
        torch.cuda.synchronize()
        for j in range(len(shapes)):
            yref, absY = refs[j]
            assert_within(ys[j].cpu().numpy()[None], yref, absY, what=f"stage {j} run {rep}")
    assert chain.failed_waits() == 0
    chain.close()


def test_chain_rejects_bad_stages():
    _, _, pc, ps = make(1, 64, 256, tid=300)
    x = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(64, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.Chain([(1, 64, 200, pc, ps, x, y, 0)])
    assert e.value.status == lb.E_SHAPE
    _, _, pc2, ps2 = make(2, 64, 256, tid=302)
    with pytest.raises(lb.LowbitError) as e:
        lb.Chain([(1, 64, 256, pc, ps, x, y, 0), (2, 64, 256, pc2, ps2, x, y, 1)])
    assert e.value.status == lb.E_UNSUPPORTED
    with pytest.raises(lb.LowbitError) as e:
        lb.Chain([(1, 64, 256, pc, ps, x, y, 0)], x_dtype=lb.I8)
    assert e.value.status == lb.E_UNSUPPORTED


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("F,K", [(640, 1024), (256, 17408)])
@pytest.mark.parametrize("with_down", [False, True])
def test_chain_silu_mul_epilogue(fmt, dt, F, K, with_down):
    """A fused gate/up stage with the SiLU-mul epilogue writes F values
    z = silu(g) u; alone it runs in the streaming kernel, followed by a
    waiting down projection (x = z) in the dependent kernel.  z must meet the
    tolerance propagated from the product tolerance of g and u; the down
    stage must match the oracle applied to the GPU's own z."""
    xdt = lb.F32 if dt == "f32" else lb.BF16
    cg = codes_for(fmt, SEED, 400 + F % 7, F, K)
    cu = codes_for(fmt, SEED, 410 + F % 7, F, K)
    sg = synth.group_scales(SEED, 420, F, K // 128)
    su = synth.group_scales(SEED, 421, F, K // 128)
    fused_c, fused_s = O.fuse_gate_up(cg, cu), O.fuse_gate_up(sg, su)
    pc, ps = lb.pack(fmt, dev(fused_c), dev(fused_s.view(np.int16)))
    if dt == "f32":
        xh = synth.normal_f32(SEED, 430, 1, K)
        x = dev(xh)[0]
        xkind = O.X_F32
    else:
        xh = synth.normal_bf16(SEED, 430, 1, K)
        x = dev(xh.view(np.int16)).view(torch.bfloat16)[0]
        xkind = O.X_BF16
    gref, absG = O.matmul(cg, sg, xkind, xh)
    uref, absU = O.matmul(cu, su, xkind, xh)
    gref, absG, uref, absU = gref[0], absG[0], uref[0], absU[0]
    zref = O.silu_mul(gref, uref)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    z = torch.full((F,), float("nan"), device="cuda", dtype=tdt)
    stages = [(fmt, 2 * F, K, pc, ps, x, z, 0, lb.EPI_SILU_MUL)]
    if with_down:
        Nd = 384
        cd = codes_for(fmt, SEED, 440, Nd, F)
        sd = synth.group_scales(SEED, 441, Nd, F // 128)
        pcd, psd = lb.pack(fmt, dev(cd), dev(sd.view(np.int16)))
        yd = torch.full((Nd,), float("nan"), device="cuda", dtype=tdt)
        stages.append((fmt, Nd, F, pcd, psd, z, yd, 1))
    chain = lb.Chain(stages, x_dtype=xdt, y_dtype=xdt)
    for rep in range(3):
        z.fill_(float("nan"))
        if with_down:
            yd.fill_(float("nan"))
        chain.run()
        torch.cuda.synchronize()
        zg = to_np(z)
        tol = silu_mul_tolerance(gref, uref, absG, absU, zref, dt == "bf16")
        err = np.abs(zg - zref)
        assert np.all(np.isfinite(zg)), f"run {rep}: non-finite z"
        assert np.all(err <= tol), f"run {rep}: z error {np.max(err / tol):.3g} x tolerance"
        if with_down:
            if dt == "f32":
                zin, kind = zg.astype(np.float32)[None], O.X_F32
            else:
                zin, kind = z.view(torch.int16).cpu().numpy().view(np.uint16)[None], O.X_BF16
            ydr, absYd = O.matmul(cd, sd, kind, zin)
            assert_within(to_np(yd)[None], ydr, absYd, bf16_out=dt == "bf16", what=f"down run {rep}")
    assert chain.failed_waits() == 0
    chain.close()


def test_chain_epilogue_rejects():
    _, _, pc, ps = make(1, 72, 256, tid=450)
    x = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(72, device="cuda")
    with pytest.raises(lb.LowbitError) as e:  # 72 rows: not whole 16-row blocks
        lb.Chain([(1, 72, 256, pc, ps, x, y, 0, lb.EPI_SILU_MUL)])
    assert e.value.status == lb.E_SHAPE
    _, _, pc, ps = make(1, 64, 256, tid=452)
    with pytest.raises(lb.LowbitError) as e:
        lb.Chain([(1, 64, 256, pc, ps, x, y, 0, 7)])
    assert e.value.status == lb.E_UNSUPPORTED


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("wait", [0, 1])
@pytest.mark.parametrize("rows", [2, 5, 8])
def test_chain_rows(fmt, wait, rows):
    """Chains of small-M products (every stage takes rows x K activations):
    each row of each stage within the oracle tolerance, on ragged N, K from
    one group to 136 groups, and on repeated runs.  Ternary rows with bf16
    activations take three split terms each, so at most five rows."""
    shapes = [(640, 1024), (100, 5120), (256, 17408), (48, 128), (3000, 2560)]
    if fmt != 1 and rows > 5:
        _, _, pc, ps = make(fmt, 64, 256, tid=498)
        x = torch.zeros((rows, 256), dtype=torch.bfloat16, device="cuda")
        y = torch.zeros((rows, 64), device="cuda")
        with pytest.raises(lb.LowbitError) as e:
            lb.Chain([(fmt, 64, 256, pc, ps, x, y, wait)], x_dtype=lb.BF16, rows=rows)
        assert e.value.status == lb.E_SHAPE
        return
    mats, xs, ys, refs = [], [], [], []
    for j, (N, K) in enumerate(shapes):
        codes, scales, pc, ps = make(fmt, N, K, tid=500 + 2 * j)
        mats.append((pc, ps))
        xh = synth.normal_bf16(SEED, 530 + j, rows, K)
        xs.append(dev(xh.view(np.int16)).view(torch.bfloat16))
        ys.append(torch.full((rows, N), float("nan"), device="cuda"))
        refs.append(O.matmul(codes, scales, O.X_BF16, xh))
    stages = [(fmt, N, K, mats[j][0], mats[j][1], xs[j], ys[j], wait)
              for j, (N, K) in enumerate(shapes)]
    chain = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32, rows=rows)
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        chain.run()
        torch.cuda.synchronize()
        for j, (N, K) in enumerate(shapes):
            yref, absY = refs[j]
            assert_within(ys[j].cpu().numpy(), yref, absY, what=f"stage {j} run {rep}")
    assert chain.failed_waits() == 0
    chain.close()


def test_chain_rows_dependent_f32():
    """rows = 3, f32 activations: stage i reads stage i-1's [3][N] output."""
    fmt, rows = 2, 3
    dims = [1024, 640, 5120, 384]
    mats, codes, scales = [], [], []
    for j in range(len(dims) - 1):
        K, N = dims[j], dims[j + 1]
        c, s, pc, ps = make(fmt, N, K, tid=560 + 2 * j)
        mats.append((pc, ps))
        codes.append(c)
        scales.append(s)
    x0 = synth.normal_f32(SEED, 590, rows, dims[0])
    bufs = [dev(x0)] + [torch.full((rows, d), float("nan"), device="cuda") for d in dims[1:]]
    stages = [(fmt, dims[j + 1], dims[j], mats[j][0], mats[j][1], bufs[j], bufs[j + 1], 1)
              for j in range(len(dims) - 1)]
    chain = lb.Chain(stages, x_dtype=lb.F32, y_dtype=lb.F32, rows=rows)
    chain.run()
    torch.cuda.synchronize()
    outs = [b.cpu().numpy() for b in bufs]
    for j in range(len(dims) - 1):
        yref, absY = O.matmul(codes[j], scales[j], O.X_F32, outs[j].astype(np.float32))
        assert_within(outs[j + 1], yref, absY, what=f"stage {j}")
    assert chain.failed_waits() == 0
    chain.close()


def test_chain_rows_rejects():
    _, _, pc, ps = make(2, 64, 256, tid=600)
    x = torch.zeros((9, 256), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((9, 64), device="cuda")
    for rows, xdt in ((6, lb.BF16), (9, lb.BF16), (5, lb.F32), (0, lb.BF16)):
        with pytest.raises(lb.LowbitError) as e:
            lb.Chain([(2, 64, 256, pc, ps, x, y, 0)], x_dtype=xdt, rows=rows)
        assert e.value.status == lb.E_SHAPE
    with pytest.raises(lb.LowbitError) as e:  # the SiLU-mul epilogue is single-row
        lb.Chain([(2, 64, 256, pc, ps, x, y, 0, lb.EPI_SILU_MUL)], rows=2)
    assert e.value.status == lb.E_SHAPE


@pytest.mark.parametrize("N", [32752, 32768])
def test_chain_binary_codes_near_2_gib(N):
    """A binary stage of K = 524288 whose packed codes come to 2^31 - 2^20
    bytes (three row-blocks per streaming wave, 32-bit buffer offsets close
    to their limit) and to exactly 2^31 bytes (the two-row-block variant
    with 64-bit addresses).  The packed codes are raw counter words, every
    bit a fair sign, so no unpacked copy is made; sampled row-blocks are
    unpacked by the oracle and checked against its product."""
    K = 524288
    GQ, NB = K // 512, N // 16
    print(f"chain binary N={N} K={K}: {NB * GQ * 1024} code bytes", flush=True)
    pc = synth.device_u32(SEED, 301, NB * GQ * 256, "cuda").view(torch.uint8)
    ps = synth.device_scales(SEED, 302, N, K // 128, "cuda").reshape(-1)  # in packed order
    xh = synth.normal_bf16(SEED, 303, 1, K)
    x = dev(xh.view(np.int16)).view(torch.bfloat16)[0]
    y = torch.full((N,), float("nan"), device="cuda")
    chain = lb.Chain([(1, N, K, pc, ps, x, y, 0)], x_dtype=lb.BF16, y_dtype=lb.F32)
    chain.run()
    torch.cuda.synchronize()
    assert chain.failed_waits() == 0
    chain.close()
    yc = y.cpu().numpy()
    assert not np.isnan(yc).any()
    for rb in (0, 1, NB // 2 + 1, NB - 2, NB - 1):
        pcb = pc[rb * GQ * 1024:(rb + 1) * GQ * 1024].cpu().numpy()
        psb = ps[rb * GQ * 64:(rb + 1) * GQ * 64].cpu().numpy().view(np.uint16)
        codes, scales, bad = O.unpack(1, 16, K, pcb, psb)
        assert bad == 0
        yref, absY = O.matmul(codes, scales, O.X_BF16, xh)
        assert_within(yc[None, 16 * rb:16 * (rb + 1)], yref, absY, what=f"row-block {rb}")
