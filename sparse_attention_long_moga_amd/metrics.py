"""Work accounting used when reporting throughput.

Attention FLOPs count 4 * head_dim FLOPs per (query, key) pair and head: a
multiply and an add for each channel of q.k and of p.v.  With full attention
(one group) this reproduces the whole-model PFLOP figures the papernotes.org
MoGA note prints for Wan2.1-1.3B (sections 关键发现 and 消融实验表格); the test
suite checks that against the printed values.
"""


def attention_flops(pairs: int, n_heads: int, head_dim: int) -> float:
    """FLOPs of softmax(QK^T)V over `pairs` (query, key) pairs per head."""
    return 4.0 * head_dim * n_heads * float(pairs)


def moga_pairs(counts) -> int:
    """(query, key) pairs of one head of MoGA attention: the sum of n_i^2."""
    return int(sum(int(c) * int(c) for c in counts))
