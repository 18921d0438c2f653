"""CPU oracle for the sparse-attention indexer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or load this
package: only the test suite, the smoke check and the benchmark's CPU-baseline leg use
it. It shares no code, table or constant generator with the GPU library and imports
nothing from it.

It is a plain, slow, exact restatement of what the indexer computes, in float64 unless
the method fixes another precision:

* ``formats`` - bit-field decoders of e4m3 (OCP fp8), e2m1 (fp4) and e8m0 (MX scale),
  and the round-to-nearest-even quantisers the K store applies;
* ``cache``   - the byte layout of a paged K cache entry (fp8 block-flat pages and the
  MXFP4 run layout), as a writer and a reader;
* ``indexer`` - the logits I[t, s] = sum_h w[t, h] * ReLU(q[t, h, :] . k[s, :]) with each
  row's validity mask, the row ends of a paged decode / MTP step, and per-row top-k;
* ``producers`` - what feeds the path: RMSNorm and RoPE of the keys before the store,
  RoPE of the queries and the scaling of the weights;
* ``candidates`` - the two-level indexer: block scores of a source layer's logits, the
  candidate pool they select, the masked and gathered consumers and the remap of
  pool slots to positions.

Sources are the vLLM API pages ``vllm.v1.attention.ops.rocm_aiter_mla_sparse``,
``vllm.models.deepseek_v41.amd.rocm``, ``vllm.v1.attention.backends.mla.rocm_aiter_mla``
and ``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer``; each function names the
section it follows.
"""

from . import cache, candidates, formats, indexer, producers  # noqa: F401
