"""GPU parity of muon_ns_batched against the CPU float64 oracle.

Tolerances (relative Frobenius error per matrix, max over the batch): 2e-2
in bf16 compute mode, 1e-4 in fp32 compute mode.  Index and layout results
(per-head slices, megabatch slices, transposed orientation) are bitwise.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, max_rel_fro, rel_fro, storage_f64, to_dev, to_f64, torch_cuda

import newton_schulz_ns5_amd as ns

pytestmark = pytest.mark.gpu


def run_case(shape, dtype, compute, key, n_check=None, out_dtype=None):
    torch = torch_cuda()
    x = synth.gaussian(shape, key, dtype)
    xt = to_dev(x, dtype)
    out = torch.empty(shape, dtype=getattr(torch, {"bf16": "bfloat16", "f32": "float32"}[out_dtype or dtype]),
                      device="cuda")
    ns.ns_batched(xt, out, compute_dtype=compute)
    torch.cuda.synchronize()
    got = to_f64(out)
    xin = storage_f64(x, dtype)
    if len(shape) == 2:
        return rel_fro(got, oracle.newton_schulz5(xin))
    idx = range(shape[0]) if n_check is None else np.linspace(0, shape[0] - 1, n_check).astype(int)
    return max(rel_fro(got[i], oracle.newton_schulz5(xin[i])) for i in idx)


def test_c1_fp32_256():
    # One 256 x 256 N(0,1) fp32 gradient, fp32 compute.
    assert run_case((256, 256), "f32", "f32", (1, 0, 0, 1, 0)) <= TOL["f32"]


def test_c1_fp32_matches_svd_closed_form():
    torch = torch_cuda()
    x = synth.gaussian((256, 256), (1, 0, 0, 1, 0), "f32")
    out = ns.ns_batched(to_dev(x, "f32"), compute_dtype="f32")
    torch.cuda.synchronize()
    g = x.astype(np.float64)
    u, s, vt = np.linalg.svd(g)
    nrm = np.linalg.norm(g) + 1e-7
    ph = s / nrm
    for _ in range(5):
        ph = 3.4445 * ph - 4.7750 * ph ** 3 + 2.0315 * ph ** 5
    assert rel_fro(to_f64(out), (u * ph) @ vt) <= TOL["f32"]


def test_c1_bf16_mode_256():
    assert run_case((256, 256), "f32", "bf16", (1, 0, 0, 1, 0)) <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(3, 300, 520), (2, 520, 300), (2, 8, 36), (1, 384, 384), (2, 1, 5), (1, 130, 700),
                                   (3, 257, 1000)])
@pytest.mark.parametrize("compute", ["bf16", "f32"])
def test_ragged_shapes(shape, compute):
    err = run_case(shape, "bf16" if compute == "bf16" else "f32", compute, (9, shape[1], shape[2], 1, 0))
    assert err <= TOL[compute], err


def test_fp32_input_bf16_output():
    assert run_case((2, 200, 330), "f32", "bf16", (9, 1, 1, 1, 0), out_dtype="bf16") <= TOL["bf16"]


def test_zero_matrix_gives_zero():
    torch = torch_cuda()
    x = torch.zeros((2, 70, 90), dtype=torch.bfloat16, device="cuda")
    x[1].normal_()
    out = ns.ns_batched(x)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0).item()
    assert torch.isfinite(out[1].float()).all().item()


def test_in_place():
    torch = torch_cuda()
    x = to_dev(synth.gaussian((2, 128, 256), (9, 2, 2, 1, 0), "bf16"), "bf16")
    ref = ns.ns_batched(x.clone())
    ns.ns_batched(x, x)
    torch.cuda.synchronize()
    assert torch.equal(ref, x)


def test_deterministic_run_twice():
    torch = torch_cuda()
    x = to_dev(synth.gaussian((4, 256, 640), (9, 3, 3, 1, 0), "bf16"), "bf16")
    a = ns.ns_batched(x)
    b = ns.ns_batched(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_megabatch_slice_bitwise_and_parity():
    # Conv2d megabatch [64, 256, 128*3*3]: slice i alone == slice i of the batch.
    torch = torch_cuda()
    name, n, pshape = synth.conv_megabatches()[0]
    rows, cols = pshape[0], int(np.prod(pshape[1:]))
    x = synth.gaussian((n, rows, cols), (4, 0, 0, 1, 0), "bf16")
    xt = to_dev(x, "bf16")
    full = ns.ns_batched(xt)
    singles = [ns.ns_batched(xt[i]) for i in (0, 17, 63)]
    rev = ns.ns_batched(xt.flip(0).contiguous()).flip(0)
    torch.cuda.synchronize()
    for i, s in zip((0, 17, 63), singles):
        assert torch.equal(full[i], s)
    assert torch.equal(rev, full)
    xin = synth.bf16_bits_to_f64(x)
    got = to_f64(full)
    assert max_rel_fro([got[i] for i in (0, 31, 63)], [oracle.newton_schulz5(xin[i]) for i in (0, 31, 63)]) <= TOL["bf16"]


def test_megabatch_negative_control():
    # The layer-mixing view [N, out*F] gives a different result from per-slice NS.
    torch = torch_cuda()
    x = to_dev(synth.gaussian((2, 8, 36), (4, 9, 0, 1, 0), "bf16"), "bf16")
    right = ns.ns_batched(x)
    wrong = ns.ns_batched(x.reshape(1, 2, 288)).reshape(2, 8, 36)
    torch.cuda.synchronize()
    assert rel_fro(to_f64(wrong), to_f64(right)) > 0.3


def test_per_head_slice_bit_identical():
    # q_proj 4096 x 4096 viewed as 32 heads of 128 rows: heads [8, 16) run alone
    # equal the same block of the 32-head batch, bit for bit.
    torch = torch_cuda()
    q = to_dev(synth.gaussian((4096, 4096), (3, 0, 0, 1, 0), "bf16"), "bf16")
    heads = ns.per_head_view(q, 32)
    full = ns.ns_batched(heads)
    part = ns.ns_batched(heads[8:16])
    k = to_dev(synth.gaussian((1024, 4096), (3, 0, 1, 1, 0), "bf16"), "bf16")
    kf = ns.ns_batched(ns.per_head_view(k, 8))
    kp = ns.ns_batched(ns.per_head_view(k, 8)[0:8])
    torch.cuda.synchronize()
    assert torch.equal(full[8:16], part)
    assert torch.equal(kf, kp)
    xin = synth.bf16_bits_to_f64(synth.gaussian((4096, 4096), (3, 0, 0, 1, 0), "bf16"))
    got = to_f64(full)
    for h in (0, 13, 31):
        assert rel_fro(got[h], oracle.newton_schulz5(xin[h * 128:(h + 1) * 128])) <= TOL["bf16"]


def test_transpose_orientation_consistent():
    # NS(X^T) = NS(X)^T: the tall path (transposed load and store) agrees with
    # the wide path to rounding.
    torch = torch_cuda()
    x = to_dev(synth.gaussian((1, 200, 600), (9, 7, 7, 1, 0), "f32"), "f32")
    a = ns.ns_batched(x, compute_dtype="f32")
    b = ns.ns_batched(x.transpose(1, 2).contiguous(), compute_dtype="f32").transpose(1, 2)
    torch.cuda.synchronize()
    assert rel_fro(to_f64(a), to_f64(b)) < 1e-5


@pytest.mark.parametrize("shape", [(5, 128, 384), (5, 128, 4096)])
def test_max_batch_chunking_bitwise(shape):
    # Passes of at most two matrices (the input read in place pass by pass;
    # the second shape takes the split-Gram 128-row path) equal one pass.
    torch = torch_cuda()
    x = to_dev(synth.gaussian(shape, (9, 8, 8, 1, shape[2]), "bf16"), "bf16")
    a = ns.ns_batched(x)
    b = ns.ns_batched(x, max_batch=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_strided_row_views():
    # Row stride larger than cols (a column slice of a wider tensor).
    torch = torch_cuda()
    big = to_dev(synth.gaussian((2, 96, 300), (9, 9, 9, 1, 0), "bf16"), "bf16")
    view = big[:, :, 20:220]
    out = ns.ns_batched(view)
    ref = ns.ns_batched(view.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("shape", [(3, 128, 4096), (1, 128, 1024), (2, 256, 1024), (2, 384, 768)])
@pytest.mark.parametrize("steps", [5, 1])
def test_input_read_in_place_matches_copied_input(shape, steps):
    # A contiguous, aligned bf16 input that is not transposed or padded is read
    # in place by the first iteration; a row-padded view, a misaligned copy and
    # the in-place call (y == x) take the copy into the workspace.  All four
    # give the same bits.
    torch = torch_cuda()
    n, rows, cols = shape
    x = to_dev(synth.gaussian(shape, (9, 12, rows, cols, steps), "bf16"), "bf16")
    direct = ns.ns_batched(x, steps=steps)
    wide = torch.zeros((n, rows, cols + 64), dtype=x.dtype, device=x.device)
    wide[:, :, :cols] = x
    padded = ns.ns_batched(wide[:, :, :cols], steps=steps)
    flat = torch.zeros(x.numel() + 4, dtype=x.dtype, device=x.device)
    shifted = flat[4:].view(shape)          # 8 bytes past a 16-byte boundary
    shifted.copy_(x)
    mis = ns.ns_batched(shifted, steps=steps)
    inplace = x.clone()
    ns.ns_batched(inplace, inplace, steps=steps)
    torch.cuda.synchronize()
    assert torch.equal(direct, padded)
    assert torch.equal(direct, mis)
    assert torch.equal(direct, inplace)
    assert torch.equal(x, to_dev(synth.gaussian(shape, (9, 12, rows, cols, steps), "bf16"), "bf16"))  # input intact


# ---- per-iteration coefficient schedules ------------------------------------
SCHEDULE = [oracle.QUINTIC] * 4 + [(15 / 8, -10 / 8, 3 / 8)]   # four quintic steps, then the classical polynomial


@pytest.mark.parametrize("compute", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 300, 520), (1, 384, 256)])
def test_schedule_parity(shape, compute):
    torch = torch_cuda()
    dt = "bf16" if compute == "bf16" else "f32"
    x = synth.gaussian(shape, (21, shape[1], shape[2], 1, 0), dt)
    out = ns.ns_batched(to_dev(x, dt), steps=5, coeffs=SCHEDULE, compute_dtype=compute)
    torch.cuda.synchronize()
    got, xin = to_f64(out), storage_f64(x, dt)
    err = max(rel_fro(got[i], oracle.newton_schulz5(xin[i], steps=5, coeffs=SCHEDULE)) for i in range(shape[0]))
    assert err <= TOL[compute], err
    # and it is not the constant-coefficient result
    assert rel_fro(got[0], oracle.newton_schulz5(xin[0])) > 0.05


def test_constant_schedule_is_bitwise_the_scalar_path():
    torch = torch_cuda()
    xt = to_dev(synth.gaussian((2, 256, 640), (22, 0, 0, 1, 0), "bf16"), "bf16")
    a = ns.ns_batched(xt)
    b = ns.ns_batched(xt, steps=5, coeffs=[oracle.QUINTIC] * 5)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- coefficients with c = 0 ---------------------------------------------------
# With c = 0 the polynomial step is B = b A: the kernel then adds b A as an
# explicit D operand in the epilogue instead of inside the products.  The cubic
# Newton-Schulz iteration (a, b, c) = (3/2, -1/2, 0) is the textbook case.
CUBIC = (1.5, -0.5, 0.0)


@pytest.mark.parametrize("compute", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 300, 520), (1, 256, 256), (1, 640, 384), (1, 768, 1024)])
def test_cubic_coefficients_parity(shape, compute):
    # (1, 768, 1024) has 256-edge tiles (eight waves): its polynomial takes the
    # explicit D through the generic epilogue.
    torch = torch_cuda()
    dt = "bf16" if compute == "bf16" else "f32"
    x = synth.gaussian(shape, (23, shape[1], shape[2], 1, 0), dt)
    out = ns.ns_batched(to_dev(x, dt), steps=5, coeffs=CUBIC, compute_dtype=compute)
    torch.cuda.synchronize()
    got, xin = to_f64(out), storage_f64(x, dt)
    err = max(rel_fro(got[i], oracle.newton_schulz5(xin[i], steps=5, coeffs=CUBIC)) for i in range(shape[0]))
    assert err <= TOL[compute], err


def test_schedule_mixing_zero_and_nonzero_c():
    # Iterations with c = 0 (explicit D) and c != 0 (D inside the products) in one call.
    torch = torch_cuda()
    sched = [oracle.QUINTIC, CUBIC, oracle.QUINTIC, CUBIC, (15 / 8, -10 / 8, 3 / 8)]
    x = synth.gaussian((2, 512, 768), (24, 0, 0, 1, 0), "bf16")
    out = ns.ns_batched(to_dev(x, "bf16"), steps=5, coeffs=sched)
    torch.cuda.synchronize()
    got, xin = to_f64(out), storage_f64(x, "bf16")
    err = max(rel_fro(got[i], oracle.newton_schulz5(xin[i], steps=5, coeffs=sched)) for i in range(2))
    assert err <= TOL["bf16"], err


# ---- ragged 256-edge tiles ------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 1000, 3000), (1, 3000, 1000), (2, 1000, 1000)])
def test_ragged_256_edge_tiles_parity(shape):
    # Padded to 1024 x 3072 (1024 x 1024): every product has 256-edge tiles
    # (eight waves), and the last update's tiles along the real edges are
    # ragged (the generic epilogue with element stores; the tall shape writes
    # its transposed output there, the square one is stored as is).
    torch = torch_cuda()
    x = synth.gaussian(shape, (35, shape[1], shape[2], 1, 0), "bf16")
    out = ns.ns_batched(to_dev(x, "bf16"))
    torch.cuda.synchronize()
    got, xin = to_f64(out), storage_f64(x, "bf16")
    err = max(rel_fro(got[i], oracle.newton_schulz5(xin[i])) for i in range(shape[0]))
    assert err <= TOL["bf16"], err


# ---- the largest long side ------------------------------------------------------
def test_largest_long_side_parity():
    # (2^22 - 128) x 128, the longest side the library takes (a 256-row
    # operand panel of it is just under 2^31 bytes, the buffer-descriptor
    # limit), stored tall so that the load transposes it and the last update
    # writes the transposed output.  One matrix against the float64 oracle
    # (about 1.4 TFLOP of float64 work).
    torch = torch_cuda()
    n = (1 << 22) - 128
    x = synth.gaussian((n, 128), (25, 1, 0, 1, 0), "bf16")
    out = ns.ns_batched(to_dev(x, "bf16"))
    torch.cuda.synchronize()
    got = to_f64(out)
    del out
    bad = ~np.isfinite(got)
    if bad.any():  # name where the non-finite values are (rows: the long side)
        r, c = np.nonzero(bad)
        raise AssertionError(f"{bad.sum()} non-finite values in rows {r.min()}..{r.max()} "
                             f"({len(np.unique(r // 128))} 128-row blocks), columns {c.min()}..{c.max()}")
    err = rel_fro(got, oracle.newton_schulz5(storage_f64(x, "bf16")))
    assert err <= TOL["bf16"], err


def test_two_streams_get_their_own_workspace():
    # Calls enqueued on two streams at once, each with the binding's cached
    # workspace, give what the same calls give one after the other.
    torch = torch_cuda()
    xa = to_dev(synth.gaussian((4, 512, 768), (26, 0, 0, 1, 0), "bf16"), "bf16")
    xb = to_dev(synth.gaussian((4, 512, 768), (26, 1, 0, 1, 0), "bf16"), "bf16")
    ra, rb = ns.ns_batched(xa), ns.ns_batched(xb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            ya = ns.ns_batched(xa)
        with torch.cuda.stream(s2):
            yb = ns.ns_batched(xb)
        outs.append((ya, yb))
    torch.cuda.synchronize()
    for ya, yb in outs:
        assert torch.equal(ya, ra) and torch.equal(yb, rb)


# A short side of at most 256 with a long side of at least 8x it: the Gram is
# computed over K chunks whose fp32 products are summed in a fixed order
# (even and uneven chunk edges, tall and wide, 2 to 16 chunks).
@pytest.mark.parametrize("shape", [(3, 100, 2100), (2, 128, 3300), (2, 200, 2300), (1, 3000, 120), (2, 128, 8192),
                                   (1, 128, 16500)])
def test_split_k_gram_shapes(shape):
    err = run_case(shape, "bf16", "bf16", (27, shape[1], shape[2], 1, 0))
    assert err <= TOL["bf16"], err


def test_split_k_gram_batch_invariant():
    # A 128 x 4096 matrix alone and as entry 2 of a batch of 5: bitwise equal.
    torch = torch_cuda()
    x = to_dev(synth.gaussian((5, 128, 4096), (27, 1, 0, 1, 0), "bf16"), "bf16")
    full = ns.ns_batched(x)
    one = ns.ns_batched(x[2:3].clone())
    torch.cuda.synchronize()
    assert torch.equal(full[2], one[0])


def test_128_row_path_repeatable_bitwise():
    # The fused update/Gram kernel overlaps its X' stores with the next
    # sub-tiles' loads; every call of the 128-row path (Gram-only first
    # launch, fused updates, sum-and-polynomial) gives the same bits, for a
    # batch of heads and for one matrix with 256 sub-tiles per workgroup.
    torch = torch_cuda()
    for shape in ((40, 128, 4096), (1, 128, 1 << 19)):
        x = to_dev(synth.gaussian(shape, (31, shape[0], shape[2], 1, 0), "bf16"), "bf16")
        ref = ns.ns_batched(x)
        for _ in range(8):
            out = ns.ns_batched(x)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), shape
        assert not torch.isnan(ref).any()


# muon_ns_groups: several tensors in one call, every Newton-Schulz launch
# shared by all of them; each output bitwise equal to its own muon_ns_batched
# call, and the per-head q/k case against the oracle.
def test_ns_groups_per_head_q_k_bitwise_and_parity():
    torch = torch_cuda()
    qx = synth.gaussian((4096, 4096), (3, 0, 0, 1, 0), "bf16")
    kx = synth.gaussian((1024, 4096), (3, 0, 1, 1, 0), "bf16")
    qh = ns.per_head_view(to_dev(qx, "bf16"), 32)
    kh = ns.per_head_view(to_dev(kx, "bf16"), 8)
    gq, gk = ns.ns_groups([qh, kh])
    sq, sk = ns.ns_batched(qh), ns.ns_batched(kh)
    torch.cuda.synchronize()
    assert torch.equal(gq, sq) and torch.equal(gk, sk)
    qin, kin = synth.bf16_bits_to_f64(qx), synth.bf16_bits_to_f64(kx)
    gq64, gk64 = to_f64(gq), to_f64(gk)
    for h in (0, 31):
        assert rel_fro(gq64[h], oracle.newton_schulz5(qin[h * 128:(h + 1) * 128])) <= TOL["bf16"]
    for h in (0, 7):
        assert rel_fro(gk64[h], oracle.newton_schulz5(kin[h * 128:(h + 1) * 128])) <= TOL["bf16"]


@pytest.mark.parametrize("compute", ["bf16", "f32"])
def test_ns_groups_mixed_shapes_bitwise(compute):
    # wide, tall, ragged, a split-K Gram shape, a 2-D tensor, an empty one and
    # an fp32 input with a bf16 output, in one call and with max_batch = 2.
    torch = torch_cuda()
    dt = "bf16" if compute == "bf16" else "f32"
    shapes = [(3, 300, 520), (2, 520, 300), (2, 8, 36), (3, 128, 2048), (0, 64, 64)]
    xs = [to_dev(synth.gaussian(s, (31, i, 0, 1, 0), dt), dt) if s[0] else
          torch.empty(s, dtype=torch.bfloat16, device="cuda") for i, s in enumerate(shapes)]
    x2d = to_dev(synth.gaussian((200, 330), (31, 9, 0, 1, 0), "f32"), "f32")
    xs.append(x2d)
    outs = [torch.empty_like(x) for x in xs[:-1]] + [torch.empty((200, 330), dtype=torch.bfloat16, device="cuda")]
    ns.ns_groups(xs, outs, compute_dtype=compute)
    chunked = ns.ns_groups(xs, [torch.empty_like(o) for o in outs], compute_dtype=compute, max_batch=2)
    alone = [ns.ns_batched(x, torch.empty_like(o), compute_dtype=compute) for x, o in zip(xs, outs)]
    torch.cuda.synchronize()
    for o, c, a in zip(outs, chunked, alone):
        assert torch.equal(o, a) and torch.equal(c, a)
    xin = storage_f64(synth.gaussian(shapes[0], (31, 0, 0, 1, 0), dt), dt)
    assert rel_fro(to_f64(outs[0])[1], oracle.newton_schulz5(xin[1])) <= TOL[compute]


def test_ns_groups_more_problems_than_one_launch_holds():
    # Eleven problems: every phase needs two launches (at most 8 problems per
    # GEMM or poly128 launch).  Ten are 128-row heads with a split Gram (2 or
    # 3 chunks, the fused sum-and-polynomial path), one is ragged.
    torch = torch_cuda()
    shapes = [(2, 128, 2048 + 128 * (i % 3) * 4) for i in range(10)] + [(1, 300, 520)]
    xs = [to_dev(synth.gaussian(s, (33, i, 0, 1, 0), "bf16"), "bf16") for i, s in enumerate(shapes)]
    grouped = ns.ns_groups(xs)
    alone = [ns.ns_batched(x) for x in xs]
    torch.cuda.synchronize()
    for g, a in zip(grouped, alone):
        assert torch.equal(g, a)
    xin = storage_f64(synth.gaussian(shapes[9], (33, 9, 0, 1, 0), "bf16"), "bf16")
    assert rel_fro(to_f64(grouped[9])[1], oracle.newton_schulz5(xin[1])) <= TOL["bf16"]


def test_ns_groups_balanced_tile_order_bitwise():
    # One Gram launch mixes 136 tiles with K = 16384, 136 with K = 4096 and the
    # six of a 768-row matrix (K = 2048): the host then takes the balanced
    # per-XCD tile order (every XCD an equal share of every problem; six tiles
    # leave two XCDs without any).  Each matrix equals its own call (one problem
    # per launch, round order) bit for bit, and the 768 x 2048 one matches the
    # oracle.
    torch = torch_cuda()
    shapes = [(1, 4096, 16384), (1, 4096, 4096), (1, 768, 2048)]
    xs = [to_dev(synth.gaussian(s, (34, i, 0, 1, 0), "bf16"), "bf16") for i, s in enumerate(shapes)]
    grouped = ns.ns_groups(xs)
    alone = [ns.ns_batched(x) for x in xs]
    torch.cuda.synchronize()
    for g, a in zip(grouped, alone):
        assert torch.equal(g, a)
    xin = storage_f64(synth.gaussian(shapes[2], (34, 2, 0, 1, 0), "bf16"), "bf16")
    assert rel_fro(to_f64(grouped[2])[0], oracle.newton_schulz5(xin[0])) <= TOL["bf16"]


# The Frobenius normalization is folded into the first iteration (its Gram
# accumulates the unnormalized input in fp32, scaled by 1/(||U|| + eps)^2
# afterwards), so parity is checked across input scales: 1e-12 and 1e-9 (the
# norm below and near eps), 1e12 and 1e16 (||U||_F ~ 4e18, just inside the
# documented fp32 limit of 1.8e19).  The 128-row shapes take the split-Gram
# path whose norm comes from the first Gram's chunk sums of squares (the wide
# one read in place, the tall one through the transposing load).
@pytest.mark.parametrize("scale", [1e-12, 1e-9, 1e12, 1e16])
@pytest.mark.parametrize("compute", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 300, 520), (1, 520, 300), (2, 128, 2048), (2, 2048, 128)])
def test_input_scale_parity(scale, compute, shape):
    torch = torch_cuda()
    x = synth.gaussian(shape, (41, 0, 0, 1, 0), compute, std=scale)
    out = ns.ns_batched(to_dev(x, compute), compute_dtype=compute)
    torch.cuda.synchronize()
    got, xin = to_f64(out), storage_f64(x, compute)
    assert np.isfinite(got).all()
    errs = [rel_fro(got[i], oracle.newton_schulz5(xin[i])) for i in range(shape[0])]
    assert max(errs) <= TOL[compute], (scale, errs)


@pytest.mark.parametrize("shape", [(1, 256, 384), (1, 128, 2048)])
def test_input_beyond_fp32_norm_range_gives_nan(shape):
    # ||U||_F above 1.8e19 overflows the fp32 sum of squares: the documented
    # result is NaN, never a silently zero matrix (also where the norm comes
    # from the first Gram's chunk sums of squares, the 128-row shape).
    torch = torch_cuda()
    x = synth.gaussian(shape, (41, 0, 1, 1, 0), "bf16", std=1e20)
    out = ns.ns_batched(to_dev(x, "bf16"))
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
