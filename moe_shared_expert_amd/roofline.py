"""Algorithmic byte and flop counts of the shared-expert MLP, and MI355X peaks.

Algorithmic bytes are what the operation must move at minimum: the weights
once, the activations x once and the output once.  The intermediate h is an
implementation choice and is not counted.  FLOPs count the two contractions
only (2 flops per multiply-add): 2*M*H*2I for gate_up plus 2*M*I*H for down.
"""

HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak, 2.5 PFLOP/s
FP32_VALU_PEAK_TFLOPS = 157.3     # MI355X fp32 vector peak


def weight_bytes(hidden: int, inter: int, elem: int = 2) -> int:
    """gate_up [2I, H] plus down [H, I]."""
    return 3 * hidden * inter * elem


def gate_up_bytes(hidden: int, inter: int, elem: int = 2) -> int:
    return 2 * inter * hidden * elem


def down_bytes(hidden: int, inter: int, elem: int = 2) -> int:
    return hidden * inter * elem


def algorithmic_bytes(m: int, hidden: int, inter: int, in_elem: int = 2,
                      out_elem: int = 2) -> int:
    return weight_bytes(hidden, inter, in_elem) + m * hidden * in_elem + m * hidden * out_elem


def flops(m: int, hidden: int, inter: int) -> int:
    return 6 * m * hidden * inter


# Merged MLA latent projection (vLLM PR 345): y_r = x . W_r^T for one rank's column
# shard W_r [n_r, K], then the restore of the gathered [M, n] output to logical order.

def latent_projection_bytes(m: int, k: int, n_r: int, elem: int = 2, out_elem: int = 2) -> int:
    """Weight shard once, x once, the rank's output slot once."""
    return n_r * k * elem + m * k * elem + m * n_r * out_elem


def latent_restore_bytes(m: int, n: int, elem: int = 2) -> int:
    """The gathered output read once and the logical output written once."""
    return 2 * m * n * elem


def roofline_us(m: int, hidden: int, inter: int, out_elem: int = 2):
    """(bound, microseconds) of one layer at the peaks: the larger of the algorithmic
    bytes at HBM_PEAK_GBS and the flops at BF16_MFMA_PEAK_TFLOPS."""
    t_hbm = algorithmic_bytes(m, hidden, inter, 2, out_elem) / (HBM_PEAK_GBS * 1e3)
    t_mfma = flops(m, hidden, inter) / (BF16_MFMA_PEAK_TFLOPS * 1e6)
    return ("hbm", t_hbm) if t_hbm >= t_mfma else ("mfma", t_mfma)
