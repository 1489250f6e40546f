"""Closed-form storage and parameter counts (oracle, test infrastructure only).

* 4-bit codes cost 0.5 byte per parameter ([Ch. 11.3] "核心创新一").
* One fp32 constant per 64-block costs 32/64 = 0.5 bit per parameter; double
  quantization stores 8 bits per block plus one fp32 per 256 blocks:
  8/64 + 32/(64*256) bits ([Digest] "数学公式与关键细节" item 2).  The stored
  format here also keeps one fp32 offset per group, which adds another
  32/(64*256) bits.
* LoRA trainable parameters: r * (d_in + d_out) ([Repro] "LoRA 的公式和张量形状").
"""

BLOCK = 64
GROUP = 256


def constant_bits_per_param(double_quant=True, with_offset=False, block=BLOCK, group=GROUP):
    """Bits per parameter spent on quantization constants."""
    if not double_quant:
        return 32.0 / block
    bits = 8.0 / block + 32.0 / (block * group)
    if with_offset:
        bits += 32.0 / (block * group)
    return bits


def bits_per_param(double_quant=True, with_offset=True):
    """Total storage bits per weight: 4-bit code + constants."""
    return 4.0 + constant_bits_per_param(double_quant, with_offset)


def first_level_constant_bytes(n_params, block=BLOCK):
    """Bytes of fp32 block constants without double quantization."""
    return (n_params // block) * 4


def dq_saving_bytes(n_params, with_offset=False):
    """Bytes saved by double quantization versus fp32 block constants."""
    saved_bits = constant_bits_per_param(False) - constant_bits_per_param(True, with_offset)
    return n_params * saved_bits / 8.0


def code_bytes(n_params):
    """Bytes of packed 4-bit codes."""
    return n_params // 2


def lora_param_count(r, d_in, d_out):
    """Trainable LoRA parameters of one linear: A [r, d_in] plus B [d_out, r]."""
    return r * (d_in + d_out)


def stored_bytes(d_out, d_in):
    """Exact bytes of the stored NF4 + DQ weight: codes, int8 constants, fp32 scale and offset."""
    n = d_out * d_in
    n_blocks = n // BLOCK
    n_groups = (n_blocks + GROUP - 1) // GROUP
    return n // 2 + n_blocks + 8 * n_groups
