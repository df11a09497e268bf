"""Plain, slow fp64 CPU oracle of the indexer -> Top-K -> sparse-MLA-attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import or call anything in this package.  It shares no code with the
HIP library or its Python binding and imports neither.

What it computes (each function cites the passage it follows; the pages are the five
"Day-0 adaptation" articles, the method being the sparse-attention chain described in
"Day 0 Support for New LLM Architectures", Step 1 and Key Optimization 1):

  * codecs: OCP E4M3FN decode table and round-to-nearest-even encoder; bf16 bit decode.
  * A0: per-(token, head) power-of-two scale for quantising the indexer query to e4m3.
  * scores  S[t,s] = sum_h w[t,h] * max(0, q_I[t,h] . k_I[s])   for s <= p_t  (fp64).
  * Top-K   the k_t = min(K, p_t+1) largest scores under (score desc, position asc),
            emitted in ascending position order, padded with -1.
  * attention  softmax(scale * q . c_s) over the selected rows c_s of the latent cache,
            applied to the first D_v dims of the same rows; lse in natural log (fp64).
  * cache append  new rows written into their page slots: e4m3 with a per-token fp32 scale
            amax/448 (codes: RNE of the fp32 quotient, clamped to +-448), MXFP8 (below), or
            bf16 RNE.
  * blocks  block-granular selection: a 64-position page scores the largest token score among
            its causal positions; the K/64 best pages are kept (score desc, page asc) and
            expanded to their causal positions.
  * MXFP8   the indexer's Q and K quantised per 32 consecutive elements with a shared
            power-of-two scale 2^X, X = floor(log2 amax) - 8, codes RNE(x / 2^X) clamped to
            +-448; scores then use the decoded values.

Pins (see tests/test_oracle_*.py): the codec table against the spec's fixed points and
torch's casts; A0 against a brute-force search of powers of two; scores against a loop
implementation and hand-worked closed forms; Top-K against the rank definition and
invariants; attention against a loop implementation of dense causal attention (K >= n),
the K = 1 and equal-row special cases and the equal-logit lse closed form; the per-token
quantiser against torch's float8 cast, hand-worked rows and its error bound; the MXFP8
quantiser against a brute-force exponent search, torch's float8 cast, hand-worked groups, its
error bound, and integer inputs that it must represent exactly; block selection against a
brute-force page scan, hand-worked rows and its equivalence with walking the token ranking
until K/64 distinct pages are met.
"""
from .codecs import (E4M3_TABLE, e4m3_decode, e4m3_round, e4m3_encode, bf16_decode,
                     bf16_round)
from .method import (a0_scale, a0_quantize, token_scores, topk_token, sparse_mla_token,
                     decode_rows, quantize_row_e4m3, cache_append, mx_scale_exponent,
                     mx_quantize, mx_decode, mx_quantize_query, MX_GROUP, block_scores,
                     topk_blocks, expand_blocks, Oracle)
from . import brute

__all__ = ["E4M3_TABLE", "e4m3_decode", "e4m3_round", "e4m3_encode", "bf16_decode",
           "bf16_round", "a0_scale", "a0_quantize", "token_scores", "topk_token",
           "sparse_mla_token", "decode_rows", "quantize_row_e4m3", "cache_append",
           "mx_scale_exponent", "mx_quantize", "mx_decode", "mx_quantize_query", "MX_GROUP",
           "block_scores", "topk_blocks", "expand_blocks", "Oracle", "brute"]
