"""fp64 CPU oracle for the DiT self-attention path (test infrastructure).

This package is test infrastructure, not product code. Only the test suite,
the package smoke check and the benchmark's CPU-baseline leg may import it.
It shares no code with the HIP library: it is a plain NumPy float64
restatement of what the path computes, written from the pages' definitions.

What each function follows (pages are cited by title and section):
  * rope_tables / rope_split_halves / rope_interleaved /
    interleaved_to_split_permutation -- Difflet PR #153 "TPU sequence
    parallelism ...", the FLUX split-RoPE commit (channels permuted once to
    [0, 2, ..., 1, 3, ...], which turns the pair rotation into slicing and
    concatenation; q.k is unchanged when both get the same permutation) and the Wan
    padding + split RoPE commit (pad rows get the identity rotation). The
    per-axis frequency schedule is not printed on the pages; the plain
    reading used here is the standard 1-D schedule theta^(-2j/c_a) per axis
    over that axis's own channel count, axes concatenated in pair space.
  * rms_norm -- the per-head q/k RMS normalisation with a weight vector that
    precedes RoPE (Difflet PR #153: the FLUX and Wan split-RoPE commits
    permute the q/k RMSNorm weights along with the channels).
  * attention -- softmax(scale * Q K^T) V over the valid keys only, with the
    natural-log log-sum-exp per query row (mstar PR #376: the ragged
    attention call can also hand back each row's log-sum-exp, fp32, natural
    log). Pad keys are dropped
    exactly (Difflet PR #153, Wan padding commit; maxdiffusion PR #491, the
    ragged KV tail carries the real length). Pad query rows give O = 0 and
    LSE = -inf (a convention: -inf is the merge's identity).
  * segment_valid_rows / attention_segmented -- sequences cut into segments
    that are each padded at their own tail (maxdiffusion PR #491: with ring
    parallelism every segment gets its own tail padding, and the padding
    descriptor holds the real length and the number of segments), attended as
    one softmax over every real key.
  * fixed_m_bound -- the a-priori row-max bound of the fixed-m softmax
    (maxdiffusion PR #491: fixed-m metadata from norm reductions and the key
    mean over the real rows, with an online-softmax fallback). The formula
    is not printed on the pages; the plain Cauchy-Schwarz reading
    scale * (q.kbar + |q| max_j |k_j - kbar|) is used.
  * lse_merge -- combining per-key-shard (O, LSE) pairs into the single-pass
    result (mstar PR #376, attention_over_sharded_keys).
  * pad_tokens / unpad_tokens / plan_padding -- tail padding of token rows to
    a multiple (Difflet PR #153 Wan padding commit, 4680 -> 4736;
    maxdiffusion PR #491 lane padding, 75,600 -> 75,776 at CP=4).
  * attention_bruteforce -- the same definition in pure-Python loops for
    tiny sizes, used only to cross-check `attention`.
"""
from .reference import (  # noqa: F401
    bf16_to_f64,
    plan_padding,
    pad_tokens,
    unpad_tokens,
    rope_pair_frequencies,
    rope_tables,
    rope_split_halves,
    rope_interleaved,
    interleaved_to_split_permutation,
    rms_norm,
    attention,
    attention_bruteforce,
    segment_valid_rows,
    attention_segmented,
    fixed_m_bound,
    lse_merge,
    dit_path,
)
