"""The C ABI on the host: the library loads, exports what include/moe.h declares, and
rejects bad arguments before touching the GPU (these calls never reach HIP)."""
import os
import re
import subprocess

import pytest

import mixture_experts_layer_gemv_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
FAKE = 1 << 20  # an aligned non-NULL address; never dereferenced by the argument checks


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    assert names == sorted(moe.SIGNATURES), names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z_]+)\b", out))
    missing = set(declared_functions()) - exported
    assert not missing, missing
    lib = moe.lib()
    for name in declared_functions():
        assert getattr(lib, name) is not None


def test_abi_version():
    assert moe.abi_version() == 1


def rc_forward(**kw):
    args = dict(x=FAKE, router_w=FAKE, w_gate=FAKE, w_up=FAKE, w_down=FAKE, scales=FAKE, pad_mask=None,
                out=FAKE, T=8, d=256, f=512, E=8, k=2)
    args.update(kw)
    lib = moe.lib()
    return lib.moe_forward(args["x"], args["router_w"], args["w_gate"], args["w_up"], args["w_down"],
                           args["scales"], args["pad_mask"], args["out"], args["T"], args["d"], args["f"],
                           args["E"], args["k"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(x=None), moe.MOE_ERR_INVALID, "x is NULL"),
    (dict(out=None), moe.MOE_ERR_INVALID, "out is NULL"),
    (dict(w_down=None), moe.MOE_ERR_INVALID, "w_down is NULL"),
    (dict(x=FAKE + 2), moe.MOE_ERR_INVALID, "aligned"),
    (dict(T=-1), moe.MOE_ERR_INVALID, "T must be"),
    (dict(d=0), moe.MOE_ERR_INVALID, "> 0"),
    (dict(k=0), moe.MOE_ERR_INVALID, "> 0"),
    (dict(k=9), moe.MOE_ERR_INVALID, "k must be <= E"),
    (dict(E=65, k=2), moe.MOE_ERR_UNSUPPORTED, "E > 64"),
    (dict(d=200), moe.MOE_ERR_UNSUPPORTED, "multiples of 256"),
    (dict(f=320), moe.MOE_ERR_UNSUPPORTED, "multiples of 256"),
    (dict(T=1 << 24, k=2), moe.MOE_ERR_UNSUPPORTED, "2^24"),
    # one expert's matrix must stay below 2^31 bytes (32-bit offsets of the weight loads)
    (dict(d=65536, f=32768), moe.MOE_ERR_UNSUPPORTED, "2^31"),
])
def test_invalid_arguments_are_rejected_before_any_launch(kw, status, msg):
    assert rc_forward(**kw) == status
    assert msg in moe.last_error()


def test_zero_tokens_is_a_no_op():
    assert rc_forward(T=0) == moe.MOE_OK


def test_stage_entry_points_check_arguments():
    lib = moe.lib()
    assert lib.moe_route(None, FAKE, None, None, FAKE, FAKE, 4, 256, 8, 2, None) == moe.MOE_ERR_INVALID
    assert lib.moe_dispatch(FAKE, None, FAKE, FAKE, FAKE, None, 4, 8, 2, None) == moe.MOE_ERR_INVALID
    assert lib.moe_dispatch(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 8, 9, None) == moe.MOE_ERR_INVALID
    assert lib.moe_down(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 4, 256, 512, 8, 2, None) == moe.MOE_ERR_INVALID
    assert "splits" in moe.last_error()
    assert lib.moe_combine(FAKE, 0, FAKE, FAKE, None, FAKE, 4, 256, 2, None) == moe.MOE_ERR_INVALID
    assert lib.moe_gate_up(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 256, 512, 8, 2, None) == moe.MOE_OK


def test_workspace_size_and_split_policy():
    # decode shapes split the down projection's contraction to fill the chip
    assert moe.down_splits(8, 6144, 32768, 8, 2) == 4
    assert moe.down_splits(64, 6144, 32768, 8, 2) == 4
    # small matrices (the tiled kernels at any T): parts of >= 128 rows while one round of
    # workgroups holds them (the tiny layer: 8 row tiles x 1 column tile -> 4 parts)
    assert moe.down_splits(64, 256, 512, 8, 2) == 4
    assert moe.down_splits(8, 1536, 2048, 8, 2) == 4
    assert moe.down_splits(100, 6144, 1024, 8, 2) == 1
    # narrow f (one GPU's share of 8-way tensor parallelism): split until the chip is filled
    assert moe.down_splits(8, 6144, 4096, 8, 2) == 4
    assert moe.down_splits(64, 6144, 4096, 8, 2) == 4
    assert moe.down_splits(8192, 6144, 4096, 8, 2) == 1
    # the policy counts the experts a batch can reach, min(E, T * k)
    assert moe.down_splits(1, 6144, 4096, 8, 2) == 4
    assert moe.down_splits(1, 6144, 32768, 8, 2) == 16  # two experts x 24 slabs: 16 parts fill the chip
    assert moe.workspace_bytes(1, 6144, 4096, 8, 2) >= 2 * 8 * 2 * 4096 * 4  # 8 gate/up parts
    # gate/up parts: about 512 workgroups of slabs x parts, parts of at least 768 rows of d
    assert moe.gate_up_parts(1, 6144, 4096, 8, 2) == 8
    assert moe.gate_up_parts(8, 6144, 4096, 8, 2) == 4
    assert moe.gate_up_parts(1, 6144, 32768, 8, 2) == 2
    assert moe.gate_up_parts(8, 6144, 32768, 8, 2) == 1
    assert moe.gate_up_parts(8192, 6144, 32768, 8, 2) == 1  # the tiled kernels
    assert moe.gate_up_parts(8, 6144, 32768, 8, 0) == 0
    # prefill, long contraction: launched with 2 or 4 parts, of which the kernel keeps fewer or all
    assert moe.down_splits(8192, 6144, 32768, 8, 2) == 2
    # 4 where one part is expected to under-fill a round of 256 workgroups (about
    # T * k / 256 + E / 2 row tiles x d / 256 column tiles) and T * k <= 8192
    assert moe.down_splits(161, 256, 8192, 8, 2) == 4
    assert moe.down_splits(768, 6144, 32768, 8, 2) == 4  # 10 x 24 tiles
    assert moe.down_splits(1024, 6144, 32768, 8, 2) == 2  # 12 x 24
    assert moe.down_splits(4096, 256, 8192, 8, 2) == 4
    assert moe.down_splits(4097, 256, 8192, 8, 2) == 2
    assert moe.down_splits(200, 256, 8448, 8, 2) == 2  # f / 128 = 66: quarters are not whole 128-row steps
    assert moe.down_splits(200, 256, 4096, 8, 2) == 1
    # up to 160 tokens matrices of at most 2^23 weights take the tiled kernels, split in parts of
    # >= 128 rows while one round of workgroups holds them (8 row tiles x 1 column tile: 16 parts)
    assert moe.down_splits(160, 256, 8192, 8, 2) == 16
    # the gate/up split's partial sums are part of the decode workspace at narrow f
    assert moe.workspace_bytes(8, 6144, 4096, 8, 2) >= 2 * 4 * 16 * 4096 * 4
    assert moe.workspace_bytes(8, 6144, 32768, 8, 2) < 16 * 32768 * 2 + 8 * 16 * 6144 * 4 + (1 << 20)
    tk = 16
    need = moe.workspace_bytes(8, 6144, 32768, 8, 2)
    assert need >= tk * 32768 * 2 + moe.down_splits(8, 6144, 32768, 8, 2) * tk * 6144 * 4
    assert moe.workspace_bytes(0, 6144, 32768, 8, 2) == 0
    assert moe.workspace_bytes(8, 65536, 32768, 8, 2) == 0  # unsupported shape
    assert moe.workspace_bytes(8, 6144, 32768, 8, 9) == 0


def test_expert_kernel_choice():
    # streaming kernels to 160 tokens only for expert matrices above 2^23 weights
    assert moe.expert_kernels(8, 6144, 32768, 8, 2) == 0
    assert moe.expert_kernels(160, 6144, 32768, 8, 2) == 0
    assert moe.expert_kernels(161, 6144, 32768, 8, 2) == 128
    assert moe.expert_kernels(384, 6144, 32768, 8, 2) == 128
    assert moe.expert_kernels(385, 6144, 32768, 8, 2) == 256
    assert moe.expert_kernels(8192, 6144, 32768, 8, 2) == 256
    assert moe.expert_kernels(8, 6144, 4096, 8, 2) == 0
    assert moe.expert_kernels(64, 256, 512, 8, 2) == 128
    assert moe.expert_kernels(160, 2048, 4096, 8, 2) == 128
    assert moe.expert_kernels(160, 2048, 4096 + 256, 8, 2) == 0
    assert moe.expert_kernels(8, 6144, 32768, 8, 0) == -1


def test_one_launch_choice(monkeypatch):
    # off unless MOE_ONE_LAUNCH=1
    monkeypatch.delenv("MOE_ONE_LAUNCH", raising=False)
    assert moe.one_launch(8, 6144, 32768, 8, 2) == 0
    monkeypatch.setenv("MOE_ONE_LAUNCH", "1")
    # T <= 64, E = 8, streaming expert kernels; not where one wavefront streams both matrices
    assert moe.one_launch(8, 6144, 32768, 8, 2) == 1
    assert moe.one_launch(64, 6144, 32768, 8, 2) == 1
    assert moe.one_launch(1, 6144, 32768, 8, 2) == 1  # split gate/up contraction
    assert moe.one_launch(2, 6144, 32768, 8, 2) == 0  # one wavefront per slab for both matrices
    assert moe.one_launch(8, 6144, 4096, 8, 2) == 1
    assert moe.one_launch(64, 6144, 4096, 8, 2) == 1
    assert moe.one_launch(65, 6144, 32768, 8, 2) == 0
    assert moe.one_launch(8, 6144, 32768, 4, 2) == 0
    assert moe.one_launch(64, 256, 512, 8, 2) == 0
    assert moe.one_launch(0, 6144, 32768, 8, 2) == 0
    assert moe.one_launch(8, 6144, 32768, 8, 0) == -1
    monkeypatch.setenv("MOE_ONE_LAUNCH", "0")
    assert moe.one_launch(8, 6144, 32768, 8, 2) == 0


def test_forward_ex_rejects_small_or_misaligned_workspace():
    lib = moe.lib()
    need = moe.workspace_bytes(8, 256, 512, 8, 2)
    base = [FAKE] * 6 + [None, FAKE, 8, 256, 512, 8, 2, None, None]
    assert lib.moe_forward_ex(*base, FAKE, need - 1, None) == moe.MOE_ERR_INVALID
    assert "too small" in moe.last_error()
    assert lib.moe_forward_ex(*base, FAKE + 16, need, None) == moe.MOE_ERR_INVALID
    assert "256-byte" in moe.last_error()


def test_split_policies_respect_the_kernels_divisibility_over_many_shapes():
    # Every supported shape gets contraction parts that the launchers accept: down parts of whole
    # 128-deep trips of f (the tiled kernels take two 64-deep slices per trip, the streaming ones
    # 32-row steps), gate/up parts (streaming kernels only) of whole 128-row blocks of d, powers
    # of two within the kernels' limits, and a workspace that holds H, the down parts and the
    # gate/up partial sums.
    checked = 0
    for d in (256, 512, 768, 1024, 2048, 4096, 6144, 8192):
        for f in (256, 512, 768, 1024, 2304, 4096, 8192, 8448, 16384, 32768):
            for E, k in ((1, 1), (2, 2), (4, 1), (8, 2), (16, 4), (64, 8)):
                for T in (1, 3, 8, 16, 17, 64, 65, 96, 97, 160, 161, 384, 385, 1024, 4096, 4097, 8192):
                    s = moe.down_splits(T, d, f, E, k)
                    g = moe.gate_up_parts(T, d, f, E, k)
                    path = moe.expert_kernels(T, d, f, E, k)
                    assert s in (1, 2, 4, 8, 16) and f % (128 * s) == 0, (T, d, f, E, k, s)
                    assert g in (1, 2, 4, 8) and d % (128 * g) == 0, (T, d, f, E, k, g)
                    assert path in (0, 128, 256), (T, d, f, E, k, path)
                    if path != 0:
                        assert g == 1, (T, d, f, E, k, g)
                    tk = T * k
                    need = tk * f * 2 + s * tk * d * 4 + (2 * g * tk * f * 4 if g > 1 else 0)
                    assert moe.workspace_bytes(T, d, f, E, k) >= need, (T, d, f, E, k)
                    checked += 1
    assert checked == 8 * 10 * 6 * 17
