"""The Python binding's own checks, without a GPU: every wrapper rejects an
operand of the wrong shape, or an output too small for what the call would
write, with ValueError before it takes a pointer, so such a buffer never
reaches a kernel.  Host tensors are used on purpose: a call that passed the
shape checks would stop at the device check instead ("must be a device
tensor"), which the last test confirms, so nothing here can launch."""
import pytest
import torch

import block_scaled_fp8_bsgemm_amd as bs

u8, f32, b16 = torch.uint8, torch.float32, torch.bfloat16


def t(*shape, dtype=u8):
    return torch.zeros(shape, dtype=dtype)


def gemm_ops(M=256, N=512, K=256):
    return t(M, K), t(M, K // 128, dtype=f32), t(N, K), t(N // 128, K // 128, dtype=f32)


def shape_error(fn, *a, **kw):
    with pytest.raises(ValueError) as e:
        fn(*a, **kw)
    assert "device tensor" not in str(e.value), str(e.value)
    return str(e.value)


def test_bsgemm_operand_shapes():
    A, sa, B, sb = gemm_ops()
    C = t(256 * 512, dtype=b16)
    shape_error(bs.bsgemm_fp8, A, sa, t(512, 128), sb, C)                       # B's K differs
    shape_error(bs.bsgemm_fp8, A, t(256, 1, dtype=f32), B, sb, C)                # a_scale [M, K/128]
    shape_error(bs.bsgemm_fp8, A, sa, B, t(2, 4, dtype=f32), C)                  # b_scale transposed
    shape_error(bs.bsgemm_fp8, A, sa.reshape(-1), B, sb, C)                      # a_scale flattened
    shape_error(bs.bsgemm_fp8, A, sa, B, sb, t(256 * 512 - 1, dtype=b16))        # C one short
    shape_error(bs.bsgemm_fp8, A, sa, B, sb, t(256 * 512, dtype=b16), bands=8,
                band_stride=32 * 512 + 64)                                       # strided bands need more
    shape_error(bs.bsgemm_fp8, A.reshape(-1), sa, B, sb, C)                      # A not 2-D


def test_mxgemm_operand_shapes():
    A, B = t(256, 256), t(512, 256)
    ea, eb = t(256, 8), t(512, 8)
    C = t(256 * 512, dtype=b16)
    shape_error(bs.mxgemm_fp8, A, t(256, 2), B, eb, C)                          # 1x128 scales
    shape_error(bs.mxgemm_fp8, A, ea, B, t(4, 8), C)                            # blockscale-shaped b
    shape_error(bs.mxgemm_fp8, A, ea, B, eb, t(100, dtype=b16))


def test_prepacked_gemm_shapes():
    A, sa, B, sb = gemm_ops()
    C = t(256 * 512, dtype=b16)
    shape_error(bs.bsgemm_fp8_pb, A, sa, t(512 * 256 - 16), sb, C)              # Bp short
    shape_error(bs.bsgemm_fp8_pb, A, t(256, 3, dtype=f32), t(512 * 256), sb, C)
    shape_error(bs.bsgemm_fp8_pb, A, sa, t(512 * 256), t(4, 3, dtype=f32), C)   # b_scale K blocks
    shape_error(bs.bprepack_e4m3, B, t(512 * 256 - 1))


def test_streaming_shapes():
    x = t(64, 256, dtype=b16)
    shape_error(bs.band_reduce, [x, t(64, 128, dtype=b16)])                     # parts differ
    shape_error(bs.band_reduce, [x, x], t(64, 255, dtype=b16))                  # out short
    shape_error(bs.band_reduce, [])
    shape_error(bs.rowq_e4m3, x, t(64, 255), t(64, dtype=f32))                  # q short
    shape_error(bs.rowq_e4m3, x, t(64, 256), t(63, dtype=f32))                  # scale short
    shape_error(bs.rowdq_e4m3, t(64, 256), t(32, dtype=f32))                    # scale rows
    shape_error(bs.rowdq_e4m3, t(64, 256), t(64, dtype=f32), t(64, 128, dtype=b16))
    shape_error(bs.band_rowq_e4m3, [x, x], t(64, 200), t(64, dtype=f32))
    shape_error(bs.band_rowq_e4m3, [x, t(32, 256, dtype=b16)])
    shape_error(bs.blockq_e4m3, t(64, 256, dtype=f32), 1, t(64, 256), t(64, 1, dtype=f32))
    shape_error(bs.blockq_e4m3, t(300, 256, dtype=f32), 128, t(300, 256), t(2, 2, dtype=f32))
    shape_error(bs.blockq_e4m3, t(64, 256, dtype=f32), 16)                      # block_rows
    shape_error(bs.actq_e4m3, x, t(64, 256), t(64, 1, dtype=f32))
    shape_error(bs.mxq_e4m3, x, t(64, 256), t(64, 7))


def test_well_formed_host_tensors_stop_at_the_device_check():
    A, sa, B, sb = gemm_ops()
    with pytest.raises(ValueError, match="device tensor"):
        bs.bsgemm_fp8(A, sa, B, sb, t(256 * 512, dtype=b16))
    with pytest.raises(ValueError, match="device tensor"):
        bs.rowq_e4m3(t(64, 256, dtype=b16), t(64, 256), t(64, dtype=f32))
