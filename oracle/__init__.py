"""CPU oracle of the quantized flash-attention forward path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute anything in this package: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code, header, table or helper with the HIP library; both
sides read the same seeded inputs from ``gen/`` and nothing else.

Every function here is a plain, slow, fp64 (numpy) statement of what one
step of the path computes, written from the four pages' description of the
method:

  * "[Feature] Sage Attention Support Varlen & write kv cache BF16/FP16"
    (PaddleNLP PR 10360): varlen batches, per-block quant of Q/K, the
    transpose/permute of V, RoPE + KV-cache write;
  * "[Refactor] Unify JIT/Customization/AOT mode" (FlashInfer PR 748): the
    batch prefill over ragged Q/K/V, the batch decode over a paged KV cache
    (indptr / indices / last-page length) with an optional log-sum-exp;
  * "KvQuantSparseFlashAttention" (Ascend ops-transformer README): the
    formula softmax(Q Dequant(K)^T / sqrt(d_k)) Dequant(V), the MLA-absorb
    mode (576 = 512 nope + 64 rope, V = K nope), per-token-head-tile-128
    scales stored inside each 656-byte cache row, block_table paging and
    sparse_indices selection;
  * "[Triton] FP8 with FA v3 API" (aiter PR 917): fp8 Q/K/V with per-head
    descales, regular and paged.

Modules:
  numerics   e4m3fn / int8 encoders, bf16 / fp16 rounding from fp64, decoders
  quant      per-head FP8 quant, per-block INT8 quant, V transpose/permute
  rope       RoPE (rotate-half) + paged KV append
  attention  prefill over a varlen batch, paged decode, sparse MLA decode,
             log-sum-exp merge of split partials
  brute      pure-Python scalar versions for tiny inputs (pins the above)

Every function is pinned by tests marked ``not gpu`` against brute force,
closed forms, library routines or invariants; see each module's header.
"""
