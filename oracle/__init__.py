"""fp64 CPU oracle for load-balanced split-KV paged decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or runs this
package; only the tests, the smoke check and the benchmark's CPU-baseline leg
do. It shares no code with the HIP path: it reads the same seeded input bytes
and computes, slowly and plainly, what the method is defined to compute.

Sources the oracle follows (cited by page title and section):

* xiaodao.ai, "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section
  "为什么 batch 越大，数字越漂亮": work is cut into 64-token tiles by live KV
  length and the global task list is spread as evenly as possible over
  persistent CTAs; long sequences take more tasks, short ones only compute what
  they have; static split-KV either fixes the split count or the split size.
* bitbyai.com, "vLLM × HPC-Ops: High-Performance Attention and MoE Backends from
  Tencent Hunyuan", section "Breaking Down the Kernels": a per-step
  load-balanced decode scheduler replacing static KV partitioning, and a fused
  prologue doing RoPE, query-key normalisation and the KV write.
* xiaodao.ai (same page), section "从实验表走到 SLA，还差一轮负载测试": the
  router GEMM keeps its top-k expert choice by splitting its fp32 weight into a
  bf16 high part and a bf16 residual, two tensor-core products summed.
* openai-hub.com, "腾讯混元HPC-Ops升级：五大算子直击推理痛点", section
  "五大算子覆盖了哪些场景": the illustrative variable-length attention call on
  a paged KV cache.

Modules:

* ``formats``   bf16 and OCP E4M3 decode/encode (OCP OFP8 spec v1.0)
* ``kv_layout`` the cache's in-page element order, element by element
* ``attention`` gather pages, then exact two-pass softmax attention; partial
                (acc, m, l) states and their log-sum-exp combination
* ``planner``   the balanced work list (bit-exact contract) and the static
                split-KV partitions used for comparison
* ``prologue``  RMSNorm, rotate-half RoPE, E4M3 quantise and paged append
* ``router``    the split-precision router GEMM (fp32 weight as bf16 high part +
                bf16 residual), exact logits, top-k, its error bound and the
                page's checks (error, greedy choice, cosine similarity)
* ``moe``       the fused FP8 MoE layer of a decode batch: per-token FP8
                quantisation, Gate-Up, SwiGLU, requantisation, Down, the
                weighted top-k merge (xiaodao.ai page, MoE paragraph of
                "为什么 batch 越大，数字越漂亮"; bitbyai.com page, MoE backend)

Parity status of every function is listed in each module's header.
"""
