"""The build's scratch guard: it reads the compiler's resource-usage remarks
and fails on a kernel whose registers spill past the limit (host logic only,
no compiler run)."""
from mixture_experts_layer_scan_amd import build as B

REMARKS = """\
gemm.hip:380:1: remark: Function Name: kernel_a [-Rpass-analysis=kernel-resource-usage]
gemm.hip:380:1: remark:     VGPRs: 187 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:380:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
  380 | __global__ void kernel_a(
      | ^
gemm.hip:380:1: remark: Function Name: kernel_b [-Rpass-analysis=kernel-resource-usage]
gemm.hip:380:1: remark:     ScratchSize [bytes/lane]: 1536 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:380:1: remark: Function Name: kernel_c [-Rpass-analysis=kernel-resource-usage]
gemm.hip:380:1: remark:     ScratchSize [bytes/lane]: 64 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_use_per_kernel():
    use = B._scratch_use(REMARKS.splitlines())
    assert use == {"kernel_a": 0, "kernel_b": 1536, "kernel_c": 64}


def test_limit_separates_spilling_kernels():
    use = B._scratch_use(REMARKS.splitlines())
    assert [f for f, b in use.items() if b > B.MAX_SCRATCH_BYTES] == ["kernel_b"]
