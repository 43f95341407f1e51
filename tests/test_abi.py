"""Host-side tests of libpsgd.so that need no GPU: the library loads and
exports every symbol include/psgd.h declares, the plan's classification,
layout and payload, and every argument error path (all of which return before
any device call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W

R = pytest.importorskip("rank_gradient_compression_amd")
B = R.binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "psgd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(psgd_[a-z_]+)\s*\(", src)) - {"psgd_reduce_fn"})


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def test_version():
    assert "gfx950" in R.psgd_version()


def views(tensors):
    rows, cols = [], []
    for _, s in tensors:
        m, n = oracle.matrix_view(s)
        rows.append(m)
        cols.append(n if len(s) >= 2 else 1)
    return rows, cols


def golden():
    out = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "payload_counts.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, r, nm, el, fl, vec = line.split()
        out[name] = tuple(int(x) for x in (r, nm, el, fl, vec))
    return out


@pytest.mark.parametrize("name,tensors", [("resnet18", W.resnet18_cifar_set()), ("lstm3", W.lstm3_wikitext_set()),
                                          ("llama7b", W.llama7b_set())])
def test_plan_matches_oracle_classification_and_payload(name, tensors):
    r, nm, el, fl, vec = golden()[name]
    rows, cols = views(tensors)
    p = R.psgd_plan_create(rows, cols, r)
    try:
        info = R.psgd_plan_get_info(p)
        assert info["ncompressed"] == nm
        assert info["dense_elems"] == el
        assert info["payload_elems"] == fl + vec
        op = oracle.Plan([s for _, s in tensors], r)
        for i in range(len(tensors)):
            kind, off, poff, qoff = R.psgd_plan_tensor(p, i)
            assert kind == op.kinds[i]
            assert off % 64 == 0
            if kind == B.PSGD_KIND_COMPRESSED:
                assert poff % 64 == 0 and qoff % 64 == 0 and poff + r * rows[i] <= info["p_elems"]
                assert qoff + r * cols[i] <= info["q_elems"]
            else:
                assert qoff == -1 and info["p_elems"] <= poff < info["p_buffer_elems"]
        assert info["flat_elems"] >= sum(a * b for a, b in zip(rows, cols))
    finally:
        R.psgd_plan_destroy(p)


def test_plan_regions_do_not_overlap():
    g = np.random.default_rng(0)
    rows = [int(x) for x in g.integers(1, 300, 40)]
    cols = [int(x) for x in g.integers(1, 300, 40)]
    p = R.psgd_plan_create(rows, cols, 3)
    try:
        info = R.psgd_plan_get_info(p)
        flat, pr, qr = [], [], []
        for i in range(40):
            kind, off, poff, qoff = R.psgd_plan_tensor(p, i)
            flat.append((off, off + rows[i] * cols[i]))
            if kind == B.PSGD_KIND_COMPRESSED:
                pr.append((poff, poff + 3 * rows[i]))
                qr.append((qoff, qoff + 3 * cols[i]))
            else:
                pr.append((poff, poff + rows[i] * cols[i]))
        for regs, limit in ((flat, info["flat_elems"]), (pr, info["p_buffer_elems"]), (qr, info["q_elems"])):
            regs.sort()
            for (a0, a1), (b0, b1) in zip(regs, regs[1:]):
                assert a1 <= b0
            assert not regs or regs[-1][1] <= limit
    finally:
        R.psgd_plan_destroy(p)


def test_caller_offsets_accepted_and_checked():
    p = R.psgd_plan_create([10, 20], [30, 1], 2, offsets=[1, 400])
    try:
        assert R.psgd_plan_tensor(p, 0)[1] == 1
        assert R.psgd_plan_get_info(p)["flat_elems"] == 420
    finally:
        R.psgd_plan_destroy(p)
    with pytest.raises(B.PsgdError) as e:
        R.psgd_plan_create([10, 20], [30, 1], 2, offsets=[0, 100])
    assert e.value.status == B.PSGD_ERR_INVALID_ARG and "overlap" in str(e.value)
    with pytest.raises(B.PsgdError):
        R.psgd_plan_create([10], [30], 2, offsets=[-1])


@pytest.mark.parametrize("rows,cols,rank,flags,status", [
    ([4], [4], 0, 0, B.PSGD_ERR_INVALID_ARG),
    ([4], [4], 65, 0, B.PSGD_ERR_UNSUPPORTED),
    ([0], [4], 1, 0, B.PSGD_ERR_INVALID_ARG),
    ([4], [-1], 1, 0, B.PSGD_ERR_INVALID_ARG),
    ([4], [4], 1, 6, B.PSGD_ERR_UNSUPPORTED),
    ([2], [1 << 30], 1, 0, B.PSGD_ERR_UNSUPPORTED),
])
def test_plan_create_errors(rows, cols, rank, flags, status):
    with pytest.raises(B.PsgdError) as e:
        R.psgd_plan_create(rows, cols, rank, flags)
    assert e.value.status == status
    assert R.psgd_last_error()


def test_empty_and_vector_only_plans():
    p = R.psgd_plan_create([], [], 4)
    info = R.psgd_plan_get_info(p)
    assert info["ntensors"] == 0 and info["flat_elems"] == 0 and info["payload_elems"] == 0
    R.psgd_plan_destroy(p)
    p = R.psgd_plan_create([5, 7], [1, 1], 2)
    info = R.psgd_plan_get_info(p)
    assert info["ncompressed"] == 0 and info["payload_elems"] == 12 and info["p_elems"] == 0
    R.psgd_plan_destroy(p)


def test_tensor_index_checked():
    p = R.psgd_plan_create([5], [6], 1)
    with pytest.raises(B.PsgdError):
        R.psgd_plan_tensor(p, 1)
    R.psgd_plan_destroy(p)


FAKE = 1 << 20  # never dereferenced: every case below fails validation first


def _compress(plan, **kw):
    a = dict(grads=FAKE, err=FAKE, mom=0, q=FAKE, pbuf=FAKE, mhat=0, hook=None, workspace=FAKE * 2,
             workspace_bytes=1 << 40)
    a.update(kw)
    opts = a.get("opts")
    R.psgd_compress(plan, a["grads"], a["err"], a["mom"], a["q"], a["pbuf"], a["mhat"], opts, a["hook"],
                    a["workspace"], a["workspace_bytes"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(grads=0), B.PSGD_ERR_INVALID_ARG),
    (dict(err=0), B.PSGD_ERR_INVALID_ARG),
    (dict(q=0), B.PSGD_ERR_INVALID_ARG),
    (dict(pbuf=0), B.PSGD_ERR_INVALID_ARG),
    (dict(grads=FAKE + 2), B.PSGD_ERR_INVALID_ARG),
    (dict(q=FAKE + 4), B.PSGD_ERR_INVALID_ARG),
    (dict(mom=FAKE), B.PSGD_ERR_INVALID_ARG),
    (dict(mhat=FAKE), B.PSGD_ERR_INVALID_ARG),  # aliases err
    (dict(workspace=0), B.PSGD_ERR_WORKSPACE),
    (dict(workspace=FAKE + 64), B.PSGD_ERR_WORKSPACE),
    (dict(workspace_bytes=16), B.PSGD_ERR_WORKSPACE),
    (dict(opts=B.step_opts(refresh_iters=-1)), B.PSGD_ERR_INVALID_ARG),
    (dict(opts=B.step_opts(power_iters=-2)), B.PSGD_ERR_INVALID_ARG),
    (dict(opts=B.step_opts(flags=64)), B.PSGD_ERR_INVALID_ARG),                     # unknown flag bit
    (dict(opts=B.step_opts(flags=B.PSGD_STEP_PAYLOAD_BF16 | B.PSGD_STEP_PAYLOAD_FP8)), B.PSGD_ERR_INVALID_ARG),
    (dict(opts=B.step_opts(flags=B.PSGD_STEP_DEFER_RESIDUAL | B.PSGD_STEP_NO_ERROR_FEEDBACK)),
     B.PSGD_ERR_INVALID_ARG),
    (dict(opts=B.step_opts(flags=B.PSGD_STEP_RESIDUAL_DEFERRED | B.PSGD_STEP_NO_ERROR_FEEDBACK)),
     B.PSGD_ERR_INVALID_ARG),
    (dict(opts=B.step_opts(params=FAKE * 4)), B.PSGD_ERR_INVALID_ARG),            # params without sgd_buf
    (dict(opts=B.step_opts(params=FAKE * 4, sgd_buf=FAKE * 4)), B.PSGD_ERR_INVALID_ARG),  # aliasing
    (dict(opts=B.step_opts(params=FAKE * 4 + 8, sgd_buf=FAKE * 8)), B.PSGD_ERR_INVALID_ARG),  # misaligned
])
def test_compress_argument_errors(kw, status):
    p = R.psgd_plan_create([64, 9], [48, 1], 2)
    try:
        if "mhat" in kw:
            kw = dict(kw, err=kw["mhat"])
        with pytest.raises(B.PsgdError) as e:
            _compress(p, **kw)
        assert e.value.status == status
    finally:
        R.psgd_plan_destroy(p)


def test_bf16_gradient_plan():
    # bfloat16 gradients: accepted alone or with momentum; the fp32 M_hat may
    # not be written over them.
    for flags in (B.PSGD_FLAG_GRADS_BF16, B.PSGD_FLAG_GRADS_BF16 | B.PSGD_FLAG_MOMENTUM):
        p = R.psgd_plan_create([64], [48], 2, flags, 0.9)
        assert R.psgd_plan_get_info(p)["flags"] == flags
        R.psgd_plan_destroy(p)
    p = R.psgd_plan_create([64, 9], [48, 1], 2, B.PSGD_FLAG_GRADS_BF16)
    try:
        with pytest.raises(B.PsgdError) as e:
            _compress(p, mhat=FAKE * 4, grads=FAKE * 4)
        assert e.value.status == B.PSGD_ERR_INVALID_ARG and "bfloat16" in str(e.value)
    finally:
        R.psgd_plan_destroy(p)


def test_momentum_plan_requires_mom():
    p = R.psgd_plan_create([64], [48], 2, B.PSGD_FLAG_MOMENTUM, 0.9)
    try:
        with pytest.raises(B.PsgdError) as e:
            _compress(p)
        assert e.value.status == B.PSGD_ERR_INVALID_ARG and "mom" in str(e.value)
    finally:
        R.psgd_plan_destroy(p)


def test_decompress_and_refresh_argument_errors():
    p = R.psgd_plan_create([64, 5], [48, 1], 2)
    try:
        for args, status in [((0, FAKE, FAKE, 8), B.PSGD_ERR_INVALID_ARG),    # M null
                             ((1, FAKE, FAKE, 8), B.PSGD_ERR_INVALID_ARG),    # vector tensor
                             ((2, FAKE, FAKE, 8), B.PSGD_ERR_INVALID_ARG),    # out of range
                             ((0, FAKE + 4, FAKE, 8), B.PSGD_ERR_INVALID_ARG),
                             ((0, FAKE, FAKE, -1), B.PSGD_ERR_INVALID_ARG)]:
            t, mptr, qptr, it = args
            if args[0] == 0 and mptr == FAKE and it == 8:
                mptr = 0
            with pytest.raises(B.PsgdError) as e:
                R.psgd_refresh(p, t, mptr, qptr, it, FAKE * 2, 1 << 40, 0)
            assert e.value.status == status, (args, e.value)
        with pytest.raises(B.PsgdError) as e:
            R.psgd_refresh(p, 0, FAKE, FAKE, 8, FAKE * 2, 16, 0)
        assert e.value.status == B.PSGD_ERR_WORKSPACE
        with pytest.raises(B.PsgdError) as e:
            R.psgd_decompress(p, FAKE, FAKE, FAKE, 0, 1 << 30, 0)
        assert e.value.status == B.PSGD_ERR_WORKSPACE
        with pytest.raises(B.PsgdError) as e:
            R.psgd_decompress(p, 0, FAKE, FAKE, FAKE * 2, 1 << 30, 0)
        assert e.value.status == B.PSGD_ERR_INVALID_ARG
    finally:
        R.psgd_plan_destroy(p)


def test_diagnostics_argument_errors():
    p = R.psgd_plan_create([64, 5], [48, 1], 2)
    qn = R.psgd_plan_get_info(p)["q_elems"]
    try:
        for args in [(0, FAKE, FAKE), (FAKE, 0, FAKE), (FAKE, FAKE * 2, 0), (FAKE, FAKE * 2, FAKE * 3 + 4)]:
            with pytest.raises(B.PsgdError) as e:
                R.psgd_step_stats(p, *args, FAKE * 4, 1 << 40, 0)
            assert e.value.status == B.PSGD_ERR_INVALID_ARG, args
        with pytest.raises(B.PsgdError) as e:
            R.psgd_step_stats(p, FAKE, FAKE * 2, FAKE * 3, 0, 1 << 40, 0)
        assert e.value.status == B.PSGD_ERR_WORKSPACE
        far = FAKE * 16
        for qa, qb, scr, out in [(0, FAKE, far, FAKE * 3), (FAKE, FAKE * 2, 0, FAKE * 3),
                                 (FAKE, FAKE * 2, far, 0), (FAKE, FAKE * 2, far, FAKE * 3 + 4),
                                 (FAKE, FAKE * 2, FAKE + 4 * (qn - 1), FAKE * 3),      # scratch over q_a
                                 (FAKE, far + 4 * qn, far, FAKE * 3)]:                 # q_b inside scratch
            with pytest.raises(B.PsgdError) as e:
                R.psgd_subspace_overlap(p, qa, qb, scr, out, FAKE * 4, 1 << 40, 0)
            assert e.value.status == B.PSGD_ERR_INVALID_ARG, (qa, qb, scr, out)
        with pytest.raises(B.PsgdError) as e:
            R.psgd_subspace_overlap(p, FAKE, FAKE * 2, far, FAKE * 3, FAKE * 4, 16, 0)
        assert e.value.status == B.PSGD_ERR_WORKSPACE
    finally:
        R.psgd_plan_destroy(p)


def test_stream_copy_argument_errors():
    with pytest.raises(B.PsgdError):
        R.psgd_stream_copy(FAKE, FAKE + 4, 16)
    with pytest.raises(B.PsgdError):
        R.psgd_stream_copy(FAKE, FAKE, 3)


@pytest.mark.parametrize("nin,nout,n,sink", [(0, 0, 16, True), (4, 1, 16, True), (1, 3, 16, True),
                                             (1, 0, 16, False), (1, 1, 6, True)])
def test_stream_probe_argument_errors(nin, nout, n, sink):
    with pytest.raises(B.PsgdError) as e:
        R.psgd_stream_probe([FAKE] * nin, [FAKE * 2] * nout, n, FAKE * 3 if sink else 0)
    assert e.value.status == B.PSGD_ERR_INVALID_ARG


def test_stream_probe_misaligned_array():
    with pytest.raises(B.PsgdError) as e:
        R.psgd_stream_probe([FAKE, FAKE + 4], [FAKE * 2], 16)
    assert e.value.status == B.PSGD_ERR_INVALID_ARG
    with pytest.raises(B.PsgdError):
        R.psgd_stream_probe([FAKE], [FAKE * 2 + 8], 16)


def test_timing_read_without_records():
    p = R.psgd_plan_create([64], [48], 2)
    ms, n = R.psgd_timing_read(p)
    assert ms == [0.0] * B.PSGD_NSTAGES and n == [0] * B.PSGD_NSTAGES
    R.psgd_timing_stages(p, 1 << B.PSGD_STAGE_RESIDUAL)  # host state only
    ms, n = R.psgd_timing_read(p)
    assert n == [0] * B.PSGD_NSTAGES
    R.psgd_plan_destroy(p)
    with pytest.raises(B.PsgdError) as e:
        R.psgd_timing_stages(0, 1)
    assert e.value.status == B.PSGD_ERR_INVALID_ARG


@pytest.mark.parametrize("q,ws,wsb,status", [
    (0, FAKE * 2, 1 << 40, B.PSGD_ERR_INVALID_ARG),
    (FAKE + 4, FAKE * 2, 1 << 40, B.PSGD_ERR_INVALID_ARG),
    (FAKE, 0, 1 << 40, B.PSGD_ERR_WORKSPACE),
    (FAKE, FAKE * 2, 16, B.PSGD_ERR_WORKSPACE),
])
def test_init_q_argument_errors(q, ws, wsb, status):
    p = R.psgd_plan_create([64, 9], [48, 1], 2)
    try:
        with pytest.raises(B.PsgdError) as e:
            R.psgd_init_q(p, q, 7, ws, wsb)
        assert e.value.status == status
    finally:
        R.psgd_plan_destroy(p)


def test_init_q_without_matrices_is_a_no_op():
    p = R.psgd_plan_create([5, 7], [1, 1], 2)
    try:
        R.psgd_init_q(p, 0, 7, FAKE * 2, 1 << 20)  # nothing to write, nothing launched
    finally:
        R.psgd_plan_destroy(p)


def test_c_client_is_built_against_the_library():
    # build() links the plain C client (csrc/c_smoke.c) with gcc against
    # libpsgd.so and the HIP runtime only; the GPU test runs it.
    import subprocess
    exe = os.path.join(os.path.dirname(R.__file__), "psgd_c_smoke")
    assert os.path.exists(exe), "build() did not produce the C client"
    out = subprocess.run(["ldd", exe], capture_output=True, text=True).stdout
    assert "libpsgd.so" in out and "libamdhip64" in out
    assert "torch" not in out and "python" not in out


def test_compress_noalloc_rejects_before_any_device_call():
    """psgd_compress_noalloc validates like psgd_compress and rejects a plan
    whose scratch exceeds the static array, all before touching a device."""
    rows, cols = views(W.llama7b_set())
    p = R.psgd_plan_create(rows, cols, 4)
    try:
        assert R.psgd_plan_get_info(p)["workspace_bytes"] > B.PSGD_NOALLOC_SCRATCH_BYTES
        with pytest.raises(B.PsgdError) as e:
            R.psgd_compress_noalloc(p, FAKE, FAKE, 0, FAKE, FAKE, 0, None, None, 0)
        assert e.value.status == B.PSGD_ERR_WORKSPACE and "static" in str(e.value)
    finally:
        R.psgd_plan_destroy(p)
    p = R.psgd_plan_create([64, 9], [48, 1], 2)
    try:
        assert R.psgd_plan_get_info(p)["workspace_bytes"] <= B.PSGD_NOALLOC_SCRATCH_BYTES
        for kw in (dict(grads=0), dict(q=FAKE + 4), dict(mom=FAKE)):
            a = dict(grads=FAKE, err=FAKE, mom=0, q=FAKE, pbuf=FAKE)
            a.update(kw)
            with pytest.raises(B.PsgdError) as e:
                R.psgd_compress_noalloc(p, a["grads"], a["err"], a["mom"], a["q"], a["pbuf"], 0, None, None, 0)
            assert e.value.status == B.PSGD_ERR_INVALID_ARG
            assert "psgd_compress_noalloc" in str(e.value)
    finally:
        R.psgd_plan_destroy(p)
