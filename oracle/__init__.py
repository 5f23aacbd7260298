"""CPU oracle for shifted short attention (S2-Attn) and bounded-history attention (HGA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package: only the
test-suite, the smoke check and the benchmark's CPU-baseline leg may call it.  It shares
no code with the HIP library; both sides are fed the same seeded bfloat16 bit patterns,
widened exactly to float64 here.

Everything is plain NumPy in float64, written from the pages' descriptions:

* ``oracle.s2attn`` -- LongLoRA's shift short attention ("LongLoRA: Efficient Fine-tuning
  of Long-Context Large Language Models", chatpaper.ai page, English abstract) as the
  LongQLoRA post describes it ("LongQLoRA: 单卡高效扩展 LLaMA2-13B 的上下文长度",
  section 03 方法介绍, Shift Short Attention paragraph and section 04 实验设置: group size
  is a quarter of the target length, used only in training).
* ``oracle.hga`` -- the bounded-history attention of "Long-Context Fine-Tuning with
  Limited VRAM" (BMW Group, English abstract): summaries of the history chunks kept in
  memory, a capped number of whole history chunks attended per query block, and
  gradients into the current segment only.

Readings taken where the pages are silent (each one is repeated where it is used):

* R1  causal order inside a shifted group is the rolled order (roll, attend causally,
      roll back).  R2 (token order inside the rolled group) is kept behind a flag.
* heads ``[H/2, H)`` are the shifted half; shift by ``G/2``; no shift when ``N == G``.
* kv head of q head ``h`` is ``floor(h * Hkv / H)``.
* logits are ``scale * q.k`` with ``scale = 1/sqrt(d)``; the diagonal is always kept.
* chunk summary = arithmetic mean of the chunk's keys, per kv head.
* chunk score = (mean of the block's queries) . summary, unscaled; top-k by score,
  ties to the lower chunk index, reported ascending with ``-1`` padding.
* one softmax over the union of the local causal keys and the selected history tokens;
  the history is detached (no gradient) and the selection is not differentiated.

Parity pins: every function here is checked against closed forms, textbook/library
special cases, brute force and finite differences by ``tests/test_oracle_*.py``.
"""
