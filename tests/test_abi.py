"""The C-ABI library loads on the CPU host and exports every declared symbol;
argument validation rejects bad calls before anything touches a device.
No compute call is made here (there is no GPU on the build host)."""
import ctypes
import os
import re

import pytest

import delayed_scaling_linear_amd as dsl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fp8_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for want in ("fp8_scale_update", "fp8_cast_transpose_amax", "fp8_linear_fwd",
                 "fp8_linear_dgrad", "fp8_linear_wgrad", "fp8_status_string", "fp8_abi_version",
                 "fp8_cast_transpose_amax_dbias", "fp8_cast_dbias_workspace_bytes",
                 "fp8_produce_cast_transpose_amax", "fp8_cast_transpose_dynamic",
                 "fp8_linear_fwd_fp8out", "fp8_cast_transpose_amax_dbias_noalloc",
                 "fp8_cast_transpose_amax_cached", "fp8_reference_copy",
                 "fp8_produce_modulate_backward", "fp8_gemm_workspace_bytes",
                 "fp8_linear_fwd_ws", "fp8_linear_dgrad_ws", "fp8_linear_wgrad_ws",
                 "fp8_cast_transpose_amax_group"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(dsl.library_path)
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_host_only_calls():
    assert dsl.fp8_abi_version() == 11
    assert dsl.fp8_status_string(0) == "FP8_OK"
    assert "SHAPE" in dsl.fp8_status_string(-2)
    assert "unknown" in dsl.fp8_status_string(-99)


def _desc(rows, cols, fmt=0, data=0x1000, data_t=0x2000, sinv=0x3000):
    return dsl._Desc(data, data_t, sinv, fmt, 0, rows, cols)


def test_validation_rejects_before_device_use():
    L = dsl.lib()
    byref = ctypes.byref
    # scale update: bad H, margin, algo, T; NULL pointers.
    assert L.fp8_scale_update(1, 1, 1, 1, 1, 4, 0, 0, 0, None) == -5
    assert L.fp8_scale_update(1, 1, 1, 1, 1, 4, 16, 200, 0, None) == -5
    assert L.fp8_scale_update(1, 1, 1, 1, 1, 4, 16, 0, 1, None) == -5
    assert L.fp8_scale_update(1, 1, 1, 1, 1, -1, 16, 0, 0, None) == -5
    assert L.fp8_scale_update(None, 1, 1, 1, 1, 4, 16, 0, 0, None) == -1
    assert L.fp8_scale_update(None, None, None, None, None, 0, 16, 0, 0, None) == 0
    # cast: shape multiples, ld, format, alignment, NULLs.
    d = _desc(32, 48)
    assert L.fp8_cast_transpose_amax(0x4000, 0, 32, 40, 48, 0x10, byref(_desc(32, 40)), 0, None, None) == -2
    assert L.fp8_cast_transpose_amax(0x4000, 0, 32, 48, 40, 0x10, byref(d), 0, None, None) == -2
    assert L.fp8_cast_transpose_amax(0x4000, 0, 32, 48, 52, 0x10, byref(d), 0, None, None) == -2
    assert L.fp8_cast_transpose_amax(0x4000, 0, 32, 48, 48, 0x10, byref(_desc(16, 48)), 0, None, None) == -2
    assert L.fp8_cast_transpose_amax(0x4000, 0, 32, 48, 48, 0x10, byref(_desc(32, 48, fmt=2)), 0, None, None) == -4
    assert L.fp8_cast_transpose_amax(0x4000, 2, 32, 48, 48, 0x10, byref(d), 0, None, None) == -5
    assert L.fp8_cast_transpose_amax(0x4001, 0, 32, 48, 48, 0x10, byref(d), 0, None, None) == -3
    assert L.fp8_cast_transpose_amax(None, 0, 32, 48, 48, 0x10, byref(d), 0, None, None) == -1
    assert L.fp8_cast_transpose_amax(0x4000, 0, 32, 48, 48, None, byref(d), 0, None, None) == -1
    assert L.fp8_cast_transpose_amax(0x4000, 0, 32, 48, 48, 0x10, byref(_desc(32, 48, data=0, data_t=0)), 0, None, None) == -1
    assert L.fp8_cast_transpose_amax(0x4000, 0, 32, 48, 48, 0x10, None, 0, None, None) == -1
    # GEMMs: K multiple of 16, output row multiple of 8, matching inner dims.
    x, w = _desc(64, 40), _desc(32, 40)
    assert L.fp8_linear_fwd(byref(x), byref(w), None, 0x5000, None) == -2
    x, w = _desc(64, 48), _desc(36, 48)
    assert L.fp8_linear_fwd(byref(x), byref(w), None, 0x5000, None) == -2
    x, w = _desc(64, 48), _desc(32, 64)
    assert L.fp8_linear_fwd(byref(x), byref(w), None, 0x5000, None) == -2
    x, w = _desc(64, 48), _desc(32, 48, fmt=3)
    assert L.fp8_linear_fwd(byref(x), byref(w), None, 0x5000, None) == -4
    x, w = _desc(64, 48), _desc(32, 48)
    assert L.fp8_linear_fwd(byref(x), byref(w), None, None, None) == -1
    assert L.fp8_linear_fwd(byref(x), byref(w), None, 0x5008, None) == -3
    assert L.fp8_linear_fwd(byref(x), byref(w), 0x6002, 0x5000, None) == -3
    assert L.fp8_linear_fwd(byref(_desc(0, 48)), byref(w), None, None, None) == 0
    # FP8-output forward: N a multiple of 16, no transposed output, shapes of y.
    def y_desc(rows, cols, fmt=1, data=0x7000, data_t=0):
        return _desc(rows, cols, fmt=fmt, data=data, data_t=data_t, sinv=0x7800)
    fwdq = L.fp8_linear_fwd_fp8out
    x, w = _desc(64, 48), _desc(40, 48)
    assert fwdq(byref(x), byref(w), None, 0x6000, byref(y_desc(64, 40)), 0x6100, None) == -2
    x, w = _desc(64, 48), _desc(32, 48)
    assert fwdq(byref(x), byref(w), None, 0x6000, byref(y_desc(64, 32, data_t=0x2000)), 0x6100,
                None) == -5
    assert fwdq(byref(x), byref(w), None, 0x6000, byref(y_desc(64, 48)), 0x6100, None) == -2
    assert fwdq(byref(x), byref(w), None, 0x6000, byref(y_desc(32, 32)), 0x6100, None) == -2
    assert fwdq(byref(x), byref(w), None, None, byref(y_desc(64, 32)), 0x6100, None) == -1
    assert fwdq(byref(x), byref(w), None, 0x6000, None, 0x6100, None) == -1
    assert fwdq(byref(x), byref(w), None, 0x6000, byref(y_desc(64, 32, fmt=2)), 0x6100,
                None) == -4
    assert fwdq(byref(x), byref(w), None, 0x6000, byref(y_desc(64, 32, data=0)), 0x6100,
                None) == -1
    assert fwdq(byref(x), byref(w), None, 0x6000, byref(y_desc(64, 32, data=0x7004)), 0x6100,
                None) == -3
    dy, wt = _desc(64, 32), _desc(32, 48)
    assert L.fp8_linear_dgrad(byref(dy), byref(_desc(48, 48)), 0x5000, None) == -2
    assert L.fp8_linear_dgrad(byref(dy), byref(_desc(32, 44)), 0x5000, None) == -2
    assert L.fp8_linear_wgrad(byref(dy), byref(_desc(64, 48)), 0x5000, 2, None) == -5
    assert L.fp8_linear_wgrad(byref(dy), byref(_desc(48, 48)), 0x5000, 1, None) == -2
    assert L.fp8_linear_wgrad(byref(_desc(40, 32)), byref(_desc(40, 48)), 0x5000, 1, None) == -2


def test_cast_group_validation():
    """The grouped cast checks every item as the single cast does, then the
    group: 1..8 items, one format, the same outputs on every non-empty item,
    no shared outputs.  Nothing reaches a device."""
    L = dsl.lib()
    G = dsl._GroupItem
    P = ctypes.POINTER(dsl._Desc)

    def items(*specs):
        descs = [d for _, d in specs]
        arr = (G * len(specs))()
        for k, ((rows, cols), d) in enumerate(specs):
            arr[k] = G(0x4000 + 0x10000 * k, rows, cols, cols, 0x10, ctypes.pointer(d), 0)
        return arr, descs

    call = lambda arr, n, src=0: L.fp8_cast_transpose_amax_group(src, arr, n, None, None)
    ok = lambda r, c, **kw: ((r, c), _desc(r, c, data=0x100000 + 0x1000 * r + c,
                                            data_t=0x200000 + 0x1000 * r + c, **kw))
    arr, keep = items(ok(32, 48))
    assert L.fp8_cast_transpose_amax_group(0, None, 1, None, None) == -1
    assert call(arr, 0) == -5
    arr9, keep9 = items(*[ok(32, 16 * (k + 1)) for k in range(9)])
    assert call(arr9, 9) == -5
    # an item's own errors: a shape not a multiple of 16, a bad source dtype
    arr, keep = items(ok(32, 48), ((32, 40), _desc(32, 40)))
    assert call(arr, 2) == -2
    arr, keep = items(ok(32, 48))
    assert call(arr, 1, src=2) == -5
    # the group's: mixed formats, mixed outputs, shared outputs
    arr, keep = items(ok(32, 48), ok(64, 48, fmt=1))
    assert call(arr, 2) == -5
    arr, keep = items(ok(32, 48), ((64, 48), _desc(64, 48, data=0x300000, data_t=0)))
    assert call(arr, 2) == -5
    arr, keep = items(((32, 48), _desc(32, 48, data=0x300000, data_t=0x310000)),
                      ((64, 48), _desc(64, 48, data=0x300000, data_t=0x320000)))
    assert call(arr, 2) == -5
    # an empty item may carry any output pointers: only empty items, no
    # scale-inverse to take -> nothing to enqueue
    arr, keep = items(((0, 48), _desc(0, 48, data=0, data_t=0, sinv=0)),
                      ((0, 16), _desc(0, 16, data=0x300000, data_t=0, sinv=0)))
    assert call(arr, 2) == 0
    with pytest.raises(ValueError):
        dsl.fp8_cast_transpose_amax_group([])


def test_split_product_workspace_validation():
    """The _ws products check what the unsplit ones check, then the
    workspace: NULL is no workspace (any size); a non-NULL one must be 16-byte
    aligned with a non-negative size.  Nothing reaches a device."""
    L = dsl.lib()
    byref = ctypes.byref
    x, w = _desc(64, 48), _desc(32, 48)
    # the unsplit checks come first
    assert L.fp8_linear_fwd_ws(byref(_desc(64, 40)), byref(_desc(32, 40)), None, 0x5000, 0x9000,
                               1 << 20, None) == -2
    assert L.fp8_linear_fwd_ws(byref(x), byref(w), None, None, 0x9000, 1 << 20, None) == -1
    # then the workspace
    assert L.fp8_linear_fwd_ws(byref(x), byref(w), None, 0x5000, 0x9008, 1 << 20, None) == -3
    assert L.fp8_linear_fwd_ws(byref(x), byref(w), None, 0x5000, 0x9000, -1, None) == -5
    dy = _desc(64, 32)
    assert L.fp8_linear_dgrad_ws(byref(dy), byref(_desc(32, 48)), 0x5000, 0x9004, 1 << 20,
                                 None) == -3
    assert L.fp8_linear_dgrad_ws(byref(dy), byref(_desc(32, 48)), 0x5000, 0x9000, -16,
                                 None) == -5
    assert L.fp8_linear_wgrad_ws(byref(dy), byref(_desc(64, 48)), 0x5000, 2, 0x9000, 1 << 20,
                                 None) == -5
    assert L.fp8_linear_wgrad_ws(byref(dy), byref(_desc(64, 48)), 0x5000, 1, 0x9002, 1 << 20,
                                 None) == -3
    # empty products return before the workspace matters
    assert L.fp8_linear_fwd_ws(byref(_desc(0, 48)), byref(w), None, None, 0x9001, -1, None) == 0
    # the size query: negative sizes are a shape error before any device query
    assert L.fp8_gemm_workspace_bytes(-1, 16, 256) == -2
    assert L.fp8_gemm_workspace_bytes(16, 16, -256) == -2
    with pytest.raises(dsl.Fp8Error):
        dsl.fp8_gemm_workspace_bytes(16, -16, 256)


def test_binding_checks_tensor_arguments():
    import torch
    with pytest.raises(ValueError):
        dsl.fp8_cast_transpose_amax(torch.zeros(16, 16, dtype=torch.bfloat16),
                                    torch.ones(1), dsl.Float8Tensor(None, None, torch.ones(1), 0, 16, 16))
    with pytest.raises(TypeError):
        dsl.fp8_cast_transpose_amax(torch.zeros(16, 16, dtype=torch.float16),
                                    torch.ones(1), dsl.Float8Tensor(None, None, torch.ones(1), 0, 16, 16))


def test_dbias_workspace_size_and_validation():
    L = dsl.lib()
    byref = ctypes.byref
    assert dsl.fp8_cast_dbias_workspace_bytes(8192, 8192) == 64 * 64 * 128 * 4
    assert dsl.fp8_cast_dbias_workspace_bytes(16, 48) == 1 * 1 * 128 * 4
    assert dsl.fp8_cast_dbias_workspace_bytes(0, 48) == 0
    assert L.fp8_cast_dbias_workspace_bytes(-1, 16) == -2
    d = _desc(32, 48)
    ws = 0x10000
    # NULL dbias, NULL / short / misaligned workspace, misaligned dbias
    assert L.fp8_cast_transpose_amax_dbias(0x4000, 0, 32, 48, 48, 0x5000, byref(d), None, None,
                                           ws, 512, None, None) == -1
    assert L.fp8_cast_transpose_amax_dbias(0x4000, 0, 32, 48, 48, 0x5000, byref(d), None, 0x6000,
                                           None, 512, None, None) == -1
    assert L.fp8_cast_transpose_amax_dbias(0x4000, 0, 32, 48, 48, 0x5000, byref(d), None, 0x6000,
                                           ws, 511, None, None) == -2
    assert L.fp8_cast_transpose_amax_dbias(0x4000, 0, 32, 48, 48, 0x5000, byref(d), None, 0x6000,
                                           ws + 8, 512, None, None) == -3
    assert L.fp8_cast_transpose_amax_dbias(0x4000, 0, 32, 48, 48, 0x5000, byref(d), None, 0x6002,
                                           ws, 512, None, None) == -3
    # the cast's own checks still apply (rows not a multiple of 16)
    d2 = _desc(30, 48)
    assert L.fp8_cast_transpose_amax_dbias(0x4000, 0, 30, 48, 48, 0x5000, byref(d2), None, 0x6000,
                                           ws, 512, None, None) == -2


def test_produce_cast_validation():
    L = dsl.lib()
    byref = ctypes.byref
    d = _desc(32, 48)
    X, A, B, Y = 0x10000, 0x20000, 0x30000, 0x40000
    ok = dict(ldx=48, lda=48, ldb=48)
    call = lambda op, ldx=48, lda=48, ldb=48, b=B, x=X, y=Y, desc=d: L.fp8_produce_cast_transpose_amax(
        op, x, ldx, A, lda, b, ldb, y, desc.rows, desc.cols, 0x5000, byref(desc), None, None, None)
    assert call(5) == -5                          # unknown op
    assert call(4, b=None) == -1                  # the finite modulation needs b too
    assert call(1, b=None) == -1                  # modulate needs b
    assert call(3, b=None) == -1                  # the two-term add needs b
    assert call(3, ldb=44) == -2
    assert call(1, ldx=40) == -2                  # ld < cols
    assert call(1, lda=52) == -2                  # ld not a multiple of 8
    assert call(1, ldb=44) == -2
    assert call(1, x=X + 8) == -3                 # misaligned input
    assert call(2, y=Y + 4) == -3                 # misaligned output
    assert call(2, desc=_desc(30, 48)) == -2      # rows not a multiple of 16


def test_dynamic_cast_validation():
    L = dsl.lib()
    byref = ctypes.byref
    d = _desc(32, 48)
    assert L.fp8_cast_transpose_dynamic(0x4000, 0, 32, 48, 48, 200, 0x5000, byref(d), 0x6000,
                                        None, None) == -5           # margin out of range
    assert L.fp8_cast_transpose_dynamic(0x4000, 0, 32, 48, 48, 0, 0x5000, byref(d), None,
                                        None, None) == -1           # amax NULL
    assert L.fp8_cast_transpose_dynamic(0x4000, 0, 32, 48, 48, 0, None, byref(d), 0x6000,
                                        None, None) == -1           # scale NULL
    d2 = _desc(32, 40)
    assert L.fp8_cast_transpose_dynamic(0x4000, 0, 32, 40, 40, 0, 0x5000, byref(d2), 0x6000,
                                        None, None) == -2           # cols not a multiple of 16


def test_binding_checks_extents_before_any_call():
    """Every descriptor and output is checked against the sizes the call
    will touch (the C ABI trusts them), before any pointer reaches it."""
    import torch
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)
    one = torch.ones(1)
    # descriptor storage that disagrees with rows / cols
    with pytest.raises(ValueError, match="data must have shape"):
        dsl.Float8Tensor(u8(16, 32), None, one, 0, 32, 16).desc()
    with pytest.raises(ValueError, match="data_t must have shape"):
        dsl.Float8Tensor(None, u8(16, 32), one, 0, 16, 32).desc()
    with pytest.raises(ValueError, match="at least one element"):
        dsl.Float8Tensor(u8(16, 32), None, torch.ones(0), 0, 16, 32).desc()
    x = dsl.Float8Tensor(u8(64, 32), None, one, 0, 64, 32)
    w = dsl.Float8Tensor(u8(48, 32), u8(32, 48), one, 0, 48, 32)
    dy = dsl.Float8Tensor(u8(64, 48), u8(48, 64), one, 1, 64, 48)
    xt = dsl.Float8Tensor(None, u8(32, 64), one, 0, 64, 32)
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="y must have shape"):
        dsl.fp8_linear_fwd(x, w, None, bf(64, 40))
    with pytest.raises(ValueError, match="bias must have shape"):
        dsl.fp8_linear_fwd(x, w, bf(40), bf(64, 48))
    with pytest.raises(ValueError, match="dx must have shape"):
        dsl.fp8_linear_dgrad(dy, w, bf(64, 48))
    with pytest.raises(ValueError, match="dw must have shape"):
        dsl.fp8_linear_wgrad(dy, xt, torch.zeros(32, 48))
    with pytest.raises(ValueError, match="bias must have shape"):
        dsl.fp8_linear_fwd_fp8out(x, w, bf(47), one, dsl.Float8Tensor(u8(64, 48), None, one, 0,
                                                                      64, 48), one)
    with pytest.raises(ValueError, match="scale_y"):
        dsl.fp8_linear_fwd_fp8out(x, w, None, torch.ones(0),
                                  dsl.Float8Tensor(u8(64, 48), None, one, 0, 64, 48), one)
    src = bf(64, 32)
    with pytest.raises(ValueError, match="scale must have"):
        dsl.fp8_cast_transpose_amax(src, torch.ones(0), x)
    with pytest.raises(ValueError, match="amax_cur must have"):
        dsl.fp8_cast_transpose_amax(src, one, x, torch.ones(0))
    with pytest.raises(ValueError, match="amax is required"):
        dsl.fp8_cast_transpose_dynamic(src, one, x, None)
    with pytest.raises(ValueError, match="amax_history must be"):
        dsl.fp8_scale_update(torch.zeros(16), one, one, one, u8(1))


def test_noalloc_dbias_validation():
    """The no-allocation entry point rejects sources whose column-sum scratch
    exceeds the fixed array, before anything is enqueued, and keeps the
    cast's own checks."""
    L = dsl.lib()
    byref = ctypes.byref
    assert dsl.NOALLOC_SCRATCH_BYTES == 4 << 20
    big = _desc(16384, 16384)                    # 128 x 128 tiles x 512 B = 8 MiB of sums
    assert dsl.fp8_cast_dbias_workspace_bytes(16384, 16384) > dsl.NOALLOC_SCRATCH_BYTES
    assert L.fp8_cast_transpose_amax_dbias_noalloc(0x4000, 0, 16384, 16384, 16384, 0x5000,
                                                   byref(big), None, 0x6000, None, None) == -8
    assert "SCRATCH" in dsl.fp8_status_string(-8)
    d = _desc(30, 48)                            # rows not a multiple of 16
    assert L.fp8_cast_transpose_amax_dbias_noalloc(0x4000, 0, 30, 48, 48, 0x5000, byref(d),
                                                   None, 0x6000, None, None) == -2
    d = _desc(32, 48)
    assert L.fp8_cast_transpose_amax_dbias_noalloc(0x4000, 0, 32, 48, 48, 0x5000, byref(d),
                                                   None, None, None, None) == -1   # dbias NULL


def test_reference_copy_and_cached_cast_validation():
    L = dsl.lib()
    byref = ctypes.byref
    assert L.fp8_reference_copy(0x1000, 0x2000, 24, 4, 0, None) == -5      # not a multiple of 16
    assert L.fp8_reference_copy(0x1000, 0x2000, 32, 0, 0, None) == -5      # no workgroups
    assert L.fp8_reference_copy(0x1000, 0x2000, 32, 4, 2, None) == -5      # bad policy
    assert L.fp8_reference_copy(None, 0x2000, 32, 4, 0, None) == -1
    assert L.fp8_reference_copy(0x1008, 0x2000, 32, 4, 0, None) == -3
    assert L.fp8_reference_copy(0x1000, 0x2000, 0, 4, 0, None) == 0       # nothing to copy
    d = _desc(30, 48)
    assert L.fp8_cast_transpose_amax_cached(0x4000, 0, 30, 48, 48, 0x5000, byref(d), None, None,
                                            None) == -2


def test_modulate_backward_validation():
    """Every rejection happens on the host before anything is enqueued."""
    L = dsl.lib()
    f = L.fp8_produce_modulate_backward
    P = [0x1000 + 0x1000 * i for i in range(7)]        # 16-byte aligned stand-ins

    def call(op=dsl.PRODUCE_MODULATE, ptrs=P, lds=(64,) * 7, rows=16, cols=64):
        args = []
        for p, ld in zip(ptrs, lds):
            args += [p, ld]
        return f(op, *args, rows, cols, None)

    assert call(op=dsl.PRODUCE_ADD) == -5                       # not a modulation
    assert call(op=dsl.PRODUCE_ADD2) == -5
    assert call(cols=60) == -2                                  # cols not a multiple of 8
    assert call(rows=-1) == -2
    assert call(lds=(64, 64, 56, 64, 64, 64, 64), cols=64) == -2   # a stride below cols
    assert call(lds=(64, 64, 64, 64, 68, 64, 64), cols=64) == -2   # a stride not a multiple of 8
    assert call(ptrs=P[:3] + [None] + P[4:]) == -1              # b NULL
    assert call(ptrs=P[:6] + [None]) == -1                      # db NULL
    assert call(ptrs=P[:1] + [0x2008] + P[2:]) == -3            # x misaligned
    assert call(rows=0) == 0 and call(cols=0) == 0              # no work
    assert call(ptrs=[None] * 7, rows=0) == 0
