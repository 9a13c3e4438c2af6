"""The C-ABI library loads, exports every function include/ssm66.h declares, and
rejects invalid arguments before touching a device.  No compute call is made
here (no GPU is needed)."""
import ctypes
import os
import re

import pytest

import selective_state_space_66_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm66.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssm_\w+)\s*\(", src, flags=re.M)))


def _header_constants():
    src = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(SSM_\w+)\s+(\d+)", src)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssm.LIB_PATH):
        from selective_state_space_66_amd import build
        build.build()
    return ssm.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == {"ssm_scan_fwd", "ssm_scan_fwd_ex", "ssm_scan_fwd_ckpt",
                          "ssm_scan_ckpt_size", "ssm_scan_bwd", "ssm_scan_bwd_ex",
                          "ssm_scan_bwd_workspace_size", "ssm_step", "ssm_ssd_fwd",
                          "ssm_conv1d_fwd", "ssm_conv1d_step", "ssm_status_string",
                          "ssm_abi_version", "ssm_scan_kernel_name", "ssm_scan_fwd_kernel",
                          "ssm_alu_probe", "ssm_scan_bwd_noalloc", "ssm_conv1d_bwd",
                          "ssm_conv1d_bwd_workspace_size"}
    raw = ctypes.CDLL(ssm.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} not exported"


def test_abi_version_and_strings(lib):
    consts = _header_constants()
    assert ssm.abi_version() == consts["SSM_ABI_VERSION"]
    for k, v in consts.items():
        if k.startswith("SSM_ERR") or k == "SSM_OK":
            s = ssm.status_string(v)
            assert s and s != "unknown status"
    assert ssm.status_string(12345) == "unknown status"


# a fake, well-aligned, never-dereferenced device address
FAKE = ctypes.c_void_p(0x10000)
MISALIGNED = ctypes.c_void_p(0x10001)


def _scan(lib, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1,
             dt_mode=0, y=FAKE, last=None, batch=2, L=8, dim=64, N=16, io=1, stream=None)
    a.update(kw)
    return lib.ssm_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                            a["softplus"], a["dt_mode"], a["y"], a["last"], a["batch"], a["L"],
                            a["dim"], a["N"], a["io"], a["stream"])


def _scan_ex(lib, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1,
             dt_mode=0, h0=None, seq_lens=None, reset=None, y=FAKE, last=None, batch=2, L=8,
             dim=64, N=16, io=1, stream=None)
    a.update(kw)
    return lib.ssm_scan_fwd_ex(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                               a["bias"], a["softplus"], a["dt_mode"], a["h0"], a["seq_lens"],
                               a["reset"], a["y"], a["last"], a["batch"], a["L"], a["dim"], a["N"],
                               a["io"], a["stream"])


def _step(lib, **kw):
    a = dict(state=FAKE, u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None,
             softplus=1, dt_mode=0, y=FAKE, batch=2, dim=64, N=16, io=1, stream=None)
    a.update(kw)
    return lib.ssm_step(a["state"], a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                        a["bias"], a["softplus"], a["dt_mode"], a["y"], a["batch"], a["dim"],
                        a["N"], a["io"], a["stream"])


@pytest.mark.parametrize("call", [_scan, _scan_ex, _step])
def test_invalid_arguments_are_rejected(lib, call):
    c = _header_constants()
    assert call(lib, N=0) == c["SSM_ERR_SHAPE"]
    assert call(lib, N=17) == c["SSM_ERR_SHAPE"]
    assert call(lib, batch=-1) == c["SSM_ERR_SHAPE"]
    assert call(lib, dim=-3) == c["SSM_ERR_SHAPE"]
    assert call(lib, io=2) == c["SSM_ERR_DTYPE"]
    assert call(lib, softplus=2) == c["SSM_ERR_FLAG"]
    assert call(lib, dt_mode=7) == c["SSM_ERR_FLAG"]
    assert call(lib, u=None) == c["SSM_ERR_NULL"]
    assert call(lib, A=None) == c["SSM_ERR_NULL"]
    assert call(lib, y=None) == c["SSM_ERR_NULL"]
    assert call(lib, u=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert call(lib, A=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert call(lib, D=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert call(lib, batch=1 << 40, dim=1 << 40) == c["SSM_ERR_SHAPE"]
    # empty work is a no-op and never reaches the device
    assert call(lib, batch=0) == c["SSM_OK"]
    assert call(lib, dim=0) == c["SSM_OK"]


def test_scan_specific_checks(lib):
    c = _header_constants()
    assert _scan(lib, L=-1) == c["SSM_ERR_SHAPE"]
    assert _scan(lib, last=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert _scan(lib, batch=1 << 20, dim=1 << 20, L=1) == c["SSM_ERR_UNSUPPORTED"]  # > 2^31 blocks
    assert _scan_ex(lib, h0=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert _scan_ex(lib, seq_lens=ctypes.c_void_p(0x10002)) == c["SSM_ERR_ALIGN"]
    assert _scan_ex(lib, L=-1) == c["SSM_ERR_SHAPE"]
    assert _scan_ex(lib, batch=1 << 20, dim=1 << 20, L=1) == c["SSM_ERR_UNSUPPORTED"]
    assert _step(lib, state=None) == c["SSM_ERR_NULL"]
    assert _step(lib, state=MISALIGNED) == c["SSM_ERR_ALIGN"]


def test_python_binding_rejects_cpu_tensors(lib):
    import torch
    u = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        ssm.scan_fwd(u, u, torch.zeros(8, 16), torch.zeros(1, 4, 16), torch.zeros(1, 4, 16))


def _conv(lib, **kw):
    a = dict(x=FAKE, w=FAKE, bias=None, silu=1, win_in=None, seq_lens=None, reset=None, out=FAKE,
             win_out=None, batch=2, L=8, dim=64, k=4, io=1, stream=None)
    a.update(kw)
    return lib.ssm_conv1d_fwd(a["x"], a["w"], a["bias"], a["silu"], a["win_in"], a["seq_lens"],
                              a["reset"], a["out"], a["win_out"], a["batch"], a["L"], a["dim"],
                              a["k"], a["io"], a["stream"])


def _conv_step(lib, **kw):
    a = dict(win=FAKE, x=FAKE, w=FAKE, bias=None, silu=1, out=FAKE, batch=2, dim=64, k=4, io=1,
             stream=None)
    a.update(kw)
    return lib.ssm_conv1d_step(a["win"], a["x"], a["w"], a["bias"], a["silu"], a["out"],
                               a["batch"], a["dim"], a["k"], a["io"], a["stream"])


@pytest.mark.parametrize("call", [_conv, _conv_step])
def test_conv_invalid_arguments_are_rejected(lib, call):
    c = _header_constants()
    assert call(lib, k=0) == c["SSM_ERR_SHAPE"]
    assert call(lib, k=5) == c["SSM_ERR_SHAPE"]
    assert call(lib, batch=-1) == c["SSM_ERR_SHAPE"]
    assert call(lib, dim=-1) == c["SSM_ERR_SHAPE"]
    assert call(lib, io=3) == c["SSM_ERR_DTYPE"]
    assert call(lib, silu=2) == c["SSM_ERR_FLAG"]
    assert call(lib, w=None) == c["SSM_ERR_NULL"]
    assert call(lib, x=None) == c["SSM_ERR_NULL"]
    assert call(lib, out=None) == c["SSM_ERR_NULL"]
    assert call(lib, x=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert call(lib, w=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert call(lib, batch=0) == c["SSM_OK"]
    assert call(lib, dim=0) == c["SSM_OK"]


def test_conv_specific_checks(lib):
    c = _header_constants()
    assert _conv(lib, L=-1) == c["SSM_ERR_SHAPE"]
    assert _conv(lib, win_out=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert _conv(lib, seq_lens=ctypes.c_void_p(0x10002)) == c["SSM_ERR_ALIGN"]
    assert _conv(lib, batch=70000) == c["SSM_ERR_UNSUPPORTED"]
    assert _conv(lib, L=64 * 65536) == c["SSM_ERR_UNSUPPORTED"]
    assert _conv_step(lib, win=None) == c["SSM_ERR_NULL"]


def _bwd(lib, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1,
             dt_mode=0, h0=None, dy=FAKE, dlast=None, du=FAKE, ddelta=FAKE, dA=FAKE, dB=FAKE,
             dC=FAKE, dD=None, dz=None, dbias=None, dh0=None, ws=ctypes.c_void_p(0x100000),
             wsb=1 << 40, batch=2, L=8, dim=64, N=16, io=1, stream=None)
    a.update(kw)
    return lib.ssm_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                            a["softplus"], a["dt_mode"], a["h0"], a["dy"], a["dlast"], a["du"],
                            a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"], a["dbias"],
                            a["dh0"], a["ws"], a["wsb"], a["batch"], a["L"], a["dim"], a["N"],
                            a["io"], a["stream"])


def test_bwd_invalid_arguments_are_rejected(lib):
    c = _header_constants()
    assert _bwd(lib, N=0) == c["SSM_ERR_SHAPE"]
    assert _bwd(lib, N=17) == c["SSM_ERR_SHAPE"]
    assert _bwd(lib, io=5) == c["SSM_ERR_DTYPE"]
    assert _bwd(lib, dt_mode=3) == c["SSM_ERR_FLAG"]
    assert _bwd(lib, dy=None) == c["SSM_ERR_NULL"]
    assert _bwd(lib, dA=None) == c["SSM_ERR_NULL"]
    assert _bwd(lib, z=FAKE, dz=None) == c["SSM_ERR_NULL"]
    assert _bwd(lib, ws=None) == c["SSM_ERR_NULL"]
    assert _bwd(lib, wsb=16) == c["SSM_ERR_SHAPE"]
    assert _bwd(lib, ws=ctypes.c_void_p(0x100040)) == c["SSM_ERR_ALIGN"]
    assert _bwd(lib, du=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert _bwd(lib, batch=0) == c["SSM_OK"]
    assert _bwd(lib, batch=1 << 20, dim=1 << 20, L=1, wsb=1 << 62) == c["SSM_ERR_UNSUPPORTED"]


def test_bwd_workspace_size(lib):
    f = lib.ssm_scan_bwd_workspace_size
    assert f(2, 40, 70, 16) >= 4 * 2 * 3 * 70 * 16  # three 16-token checkpoints per row
    assert f(-1, 4, 4, 4) == 0 and f(1, 4, 4, 17) == 0
    assert f(8, 2048, 1536, 16) > f(8, 1024, 1536, 16)


def _bwd_ex(lib, ckpt, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1,
             dt_mode=0, h0=None, lens=None, reset=None, dy=FAKE, dlast=None, du=FAKE,
             ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=None, dz=None, dbias=None, dh0=None,
             ws=ctypes.c_void_p(0x100000), wsb=1 << 40, batch=2, L=8, dim=64, N=16, io=1,
             stream=None)
    a.update(kw)
    return lib.ssm_scan_bwd_ex(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                               a["bias"], a["softplus"], a["dt_mode"], a["h0"], a["lens"],
                               a["reset"], a["dy"],
                               a["dlast"], a["du"], a["ddelta"], a["dA"], a["dB"], a["dC"],
                               a["dD"], a["dz"], a["dbias"], a["dh0"], ckpt, a["ws"], a["wsb"],
                               a["batch"], a["L"], a["dim"], a["N"], a["io"], a["stream"])


def _fwd_ckpt(lib, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1,
             dt_mode=0, h0=None, y=FAKE, last=None, ckpt=FAKE, batch=2, L=40, dim=64, N=16,
             io=1, stream=None)
    a.update(kw)
    return lib.ssm_scan_fwd_ckpt(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                 a["bias"], a["softplus"], a["dt_mode"], a["h0"], a["y"], a["last"],
                                 a["ckpt"], a["batch"], a["L"], a["dim"], a["N"], a["io"],
                                 a["stream"])


def test_training_entry_points_reject_invalid_arguments(lib):
    c = _header_constants()
    assert _fwd_ckpt(lib, ckpt=None) == c["SSM_ERR_NULL"]   # checkpoints are the point
    assert _fwd_ckpt(lib, ckpt=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert _fwd_ckpt(lib, N=17) == c["SSM_ERR_SHAPE"]
    assert _fwd_ckpt(lib, io=3) == c["SSM_ERR_DTYPE"]
    assert _fwd_ckpt(lib, u=None) == c["SSM_ERR_NULL"]
    assert _fwd_ckpt(lib, batch=0) == c["SSM_OK"]           # nothing to do, nothing launched
    assert _bwd_ex(lib, MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert _bwd_ex(lib, FAKE, dy=None) == c["SSM_ERR_NULL"]
    assert _bwd_ex(lib, FAKE, batch=0) == c["SSM_OK"]
    assert _bwd_ex(lib, FAKE, lens=MISALIGNED) == c["SSM_ERR_ALIGN"]  # int32 lengths


def test_ckpt_size(lib):
    f = lib.ssm_scan_ckpt_size
    assert f(2, 40, 70, 16) == (2 * 3 * 70 * 16 * 4 + 255) // 256 * 256  # states before 0, 16, 32
    assert f(1, 16, 8, 16) == 8 * 16 * 4 and f(1, 17, 8, 16) == 2 * 8 * 16 * 4
    assert f(-1, 4, 4, 4) == 0 and f(1, 4, 4, 17) == 0


def test_scan_kernel_choice(lib):
    """The kernel the scan picks (host logic only): the crossovers measured on
    MI355X and the degenerate sizes."""
    name = ssm.scan_kernel_name
    sixteen = ("scan_wave8_kernel / scan_wave_kernel (time-parallel, 16 lanes per row; 8 tokens per lane for bf16 "
               "io without lengths or document starts, else 4)")
    one = "scan_wave_kernel (time-parallel, one wave per row)"
    assert name(8, 2048, 1536, 16) == sixteen                          # Mamba-130M layer: 12288 rows
    assert name(8, 2048, 1535, 16) == one                              # 12280 rows
    split = ("scan_wave8_kernel (time-parallel, 16 lanes per row, 8 tokens per lane) for bf16 io without "
             "lengths or document starts, else ")
    assert name(4, 65536, 2048, 16) == split + one                     # long sequences: 8192 rows
    assert name(4, 2048, 2048, 16) == split + one
    assert name(4, 2048, 2032, 16) == one                              # 8128 rows
    assert name(4, 2048, 2047, 16) == one                              # width not a multiple of 16
    assert name(4, 2048, 2048, 8) == one                               # fewer states
    assert name(4, 200, 2048, 16) == split + "scan_fwd_kernel (sequential, 2 states per lane)"
    assert name(4, 127, 2048, 16).startswith("scan_fwd_kernel")
    assert name(8, 2048, 1536, 8) == sixteen                           # fewer states
    assert name(8, 2048, 4096, 16) == sixteen                          # Mamba-1.4B layer
    assert name(16, 2048, 2047, 16) == sixteen
    assert name(1, 2048, 1024, 16) == one                              # 1024 rows
    assert name(1, 8192, 1023, 16).startswith("scan_tpar_kernel")      # 1023 rows
    assert name(1, 128, 256, 16).startswith("scan_tpar_kernel")
    assert name(1, 127, 256, 16) == "scan_fwd_kernel (sequential, 1 state per lane)"
    assert name(8, 128, 1536, 16) == sixteen
    assert name(8, 127, 1536, 16) == "scan_fwd_kernel (sequential, 2 states per lane)"
    assert name(4, 255, 1536, 16) == "scan_fwd_kernel (sequential, 1 state per lane)"
    assert name(4, 256, 1536, 16) == one
    assert name(32, 127, 4096, 16) == "scan_fwd_kernel (sequential, 4 states per lane)"
    assert name(0, 16, 8, 16) == "none (no tokens)" and name(2, 0, 8, 16) == "none (no tokens)"
    assert name(1, 4, 4, 17) == "invalid shape" and name(-1, 4, 4, 4) == "invalid shape"
    assert name(1, 2048, 1 << 22, 16).startswith("scan_fwd_kernel")


def _scan_kernel(lib, kernel, **kw):
    """ssm_scan_fwd_kernel with fake (never dereferenced) pointers: every case
    here is rejected before any HIP call."""
    a = dict(u=FAKE, d=FAKE, A=FAKE, B=FAKE, C=FAKE, y=FAKE, batch=2, L=300, dim=48, N=16,
             io=0, ckpt=None)
    a.update(kw)
    return lib.ssm_scan_fwd_kernel(kernel, a["u"], a["d"], a["A"], a["B"], a["C"], None, None,
                                   None, 1, 0, None, None, None, a["y"], None, a["ckpt"],
                                   a["batch"], a["L"], a["dim"], a["N"], a["io"], None)


def test_forced_kernel_validation(lib):
    """ssm_scan_fwd_kernel: unknown kernels are flagged; a forced time-parallel
    kernel on a layer too wide for its 32-bit chunk offsets, and grids past the
    launch limit of the chosen kernel, are unsupported -- all before any HIP
    call."""
    c = _header_constants()
    assert c["SSM_SCAN_KERNEL_AUTO"] == 0 and c["SSM_SCAN_KERNEL_WAVE4"] == 6
    assert _scan_kernel(lib, -1) == c["SSM_ERR_FLAG"]
    assert _scan_kernel(lib, 7) == c["SSM_ERR_FLAG"]
    assert _scan_kernel(lib, c["SSM_SCAN_KERNEL_WAVE"], dim=1 << 22) == c["SSM_ERR_UNSUPPORTED"]
    assert _scan_kernel(lib, c["SSM_SCAN_KERNEL_WAVE4"], dim=1 << 22) == c["SSM_ERR_UNSUPPORTED"]
    assert _scan_kernel(lib, c["SSM_SCAN_KERNEL_TPAR"], dim=1 << 22) == c["SSM_ERR_UNSUPPORTED"]
    # four waves per row: one block per (batch, channel) row
    assert _scan_kernel(lib, c["SSM_SCAN_KERNEL_TPAR"], batch=1 << 20, dim=1 << 12, L=1) \
        == c["SSM_ERR_UNSUPPORTED"]
    # one wave per row: one block per 8 channels of a batch entry
    assert _scan_kernel(lib, c["SSM_SCAN_KERNEL_WAVE"], batch=1 << 23, dim=1 << 11, L=1) \
        == c["SSM_ERR_UNSUPPORTED"]
    # 16 lanes per row: one block per 16 channels
    assert _scan_kernel(lib, c["SSM_SCAN_KERNEL_WAVE4"], batch=1 << 24, dim=1 << 11, L=1) \
        == c["SSM_ERR_UNSUPPORTED"]
    # the automatic choice for the same shape is the sequential kernel, whose
    # blocks of 16 channels still fit
    assert ssm.scan_kernel_name(1 << 23, 1, 1 << 11, 16).startswith("scan_fwd_kernel")
    assert _scan_kernel(lib, c["SSM_SCAN_KERNEL_AUTO"], batch=1 << 23, dim=1 << 11, L=1,
                        u=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert _scan_kernel(lib, c["SSM_SCAN_KERNEL_SEQ4"], y=None) == c["SSM_ERR_NULL"]


ALIGN16 = ctypes.c_void_p(0x10000)
OFF8 = ctypes.c_void_p(0x10008)


def _ssd(lib, **kw):
    a = dict(x=ALIGN16, dt=FAKE, A=FAKE, B=ALIGN16, C=ALIGN16, D=None, z=None, bias=None,
             softplus=1, dt_mode=1, h0=None, y=ALIGN16, last=None, batch=2, L=8, H=4, P=64,
             N=128, io=1, stream=None)
    a.update(kw)
    return lib.ssm_ssd_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                           a["softplus"], a["dt_mode"], a["h0"], a["y"], a["last"], a["batch"],
                           a["L"], a["H"], a["P"], a["N"], a["io"], a["stream"])


def test_ssd_invalid_arguments_are_rejected(lib):
    c = _header_constants()
    assert _ssd(lib, batch=-1) == c["SSM_ERR_SHAPE"]
    assert _ssd(lib, P=0) == c["SSM_ERR_SHAPE"]
    assert _ssd(lib, io=4) == c["SSM_ERR_DTYPE"]
    assert _ssd(lib, dt_mode=9) == c["SSM_ERR_FLAG"]
    assert _ssd(lib, x=None) == c["SSM_ERR_NULL"]
    assert _ssd(lib, dt=None) == c["SSM_ERR_NULL"]
    assert _ssd(lib, io=0) == c["SSM_ERR_UNSUPPORTED"]   # fp32 operands: not on this kernel
    assert _ssd(lib, P=24) == c["SSM_ERR_UNSUPPORTED"]  # heads of a multiple of 16 channels
    assert _ssd(lib, N=96) == c["SSM_ERR_UNSUPPORTED"]
    assert _ssd(lib, x=OFF8) == c["SSM_ERR_ALIGN"]        # 16-byte vectors
    assert _ssd(lib, B=OFF8) == c["SSM_ERR_ALIGN"]
    assert _ssd(lib, batch=0) == c["SSM_OK"]


def test_noalloc_backward_validation(lib):
    """ssm_scan_bwd_noalloc refuses, before any HIP call, sizes whose workspace
    exceeds its static scratch, and checks its arguments like ssm_scan_bwd_ex."""
    c = _header_constants()
    limit = c["SSM_NOALLOC_SCRATCH_BYTES"]
    assert limit == 64 << 20

    def call(batch, L, dim, N, **kw):
        a = dict(u=FAKE, A=FAKE, dy=FAKE, out=FAKE, dA=FAKE, io=1)
        a.update(kw)
        return lib.ssm_scan_bwd_noalloc(a["u"], a["u"], a["A"], a["u"], a["u"], None, None, None,
                                        1, 0, None, None, None, a["dy"], None, a["out"], a["out"],
                                        a["dA"],
                                        a["out"], a["out"], None, None, None, None, None, batch,
                                        L, dim, N, a["io"], None)

    assert ssm.scan_bwd_workspace_size(4, 2048, 1536, 16) > limit
    assert call(4, 2048, 1536, 16) == c["SSM_ERR_UNSUPPORTED"]
    assert ssm.scan_bwd_workspace_size(1, 2048, 1536, 16) <= limit
    assert call(1, 2048, 1536, 16, dy=None) == c["SSM_ERR_NULL"]
    assert call(1, 2048, 1536, 16, u=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert call(1, 2048, 1536, 17) == c["SSM_ERR_SHAPE"]
    assert call(0, 2048, 1536, 16) == c["SSM_OK"]  # no rows: nothing to do, no HIP call


def test_conv_backward_validation(lib):
    """ssm_conv1d_bwd checks its arguments before any HIP call."""
    c = _header_constants()
    ws = lib.ssm_conv1d_bwd_workspace_size
    assert ws(2, 300, 64, 4) == 2 * 3 * 5 * 64 * 4   # (width + 1) sums per channel per 128 tokens
    assert ws(2, 0, 64, 4) == 2 * 1 * 5 * 64 * 4
    assert ws(2, 10, 64, 5) == 0 and ws(-1, 10, 64, 4) == 0

    def call(**kw):
        a = dict(x=FAKE, w=FAKE, bias=None, silu=1, win=None, lens=None, reset=None, dout=FAKE,
                 dwo=None, dx=FAKE, dw=FAKE, db=None, dwin=None, ws=FAKE, wsb=1 << 40, batch=2,
                 L=10, dim=64, k=4, io=1)
        a.update(kw)
        return lib.ssm_conv1d_bwd(a["x"], a["w"], a["bias"], a["silu"], a["win"], a["lens"],
                                  a["reset"], a["dout"], a["dwo"], a["dx"], a["dw"], a["db"],
                                  a["dwin"], a["ws"], a["wsb"], a["batch"], a["L"], a["dim"],
                                  a["k"], a["io"], None)

    assert call(k=0) == c["SSM_ERR_SHAPE"] and call(k=5) == c["SSM_ERR_SHAPE"]
    assert call(io=2) == c["SSM_ERR_DTYPE"]
    assert call(silu=2) == c["SSM_ERR_FLAG"]
    assert call(dw=None) == c["SSM_ERR_NULL"] and call(dout=None) == c["SSM_ERR_NULL"]
    assert call(ws=None) == c["SSM_ERR_NULL"]
    assert call(wsb=16) == c["SSM_ERR_SHAPE"]
    assert call(dx=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert call(lens=MISALIGNED) == c["SSM_ERR_ALIGN"]
    assert call(win=FAKE, dwin=FAKE) == c["SSM_ERR_FLAG"]  # not in place
    assert call(dim=0) == c["SSM_OK"]
