"""CPU oracle for the deterministic attention backward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything under ``oracle/``: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  The oracle shares no code with the HIP
path (no kernels, headers, helpers, tables or pre/post-processing).

* ``oracle.attention`` -- softmax attention forward and gradients in float64,
  written from the plain definition.
* ``oracle.schedules`` -- the DASH tile schedules (serialized baseline,
  descending-Q, shift, symmetric shift), their dQ accumulation ordinals, a
  validator and the unit-cost DAG simulator, written from the pages'
  description of the method.

Sources are cited by page title and section:
  [news]    "DASH如何革新LLM确定性训练" (pwwt.cn article)
  [summary] "Resumo Técnico: DASH – Agendamento de Atenção Determinístico para
            Treinamento de LLM de Alto Rendimento" (gist.science summary of
            arXiv 2601.21824)
"""
