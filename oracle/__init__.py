"""Plain, slow, fp64 CPU oracle of one GPU's share of a Conflux Parallelism layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  It shares no code with the HIP path (``mixed_prefill_decode_amd``)
and imports nothing from it; the HIP path never imports this package.

Pages cited (by title; sections, equations, tables and figures as printed):

* "ConfluxServe: Reconciling Resource Utilization and Parallelism Efficiency
  across Prefill and Decode in LLM Serving" -- the method: §4 (Conflux
  Parallelism execution flow, Fig. 7; KV residency, Fig. 8), §6.1 (coordinated
  attention overlap), §6.2 (Eq. 2-6), §6.3 (waterfill dispatch, dual-mode
  decode placement), §6.4 (Algorithm 1), App. B (Table 7), App. D (Eq. 7-12),
  App. E (Algorithm 2), App. F (Algorithm 3), App. G (Algorithm 4).
* "Adaptive Context Parallelism for Production LLM Serving" -- §2.1 (causal
  attention with mask M_ij = 0 for j <= i), §2.2 Eq. 1 (remaining attention
  workload R*P + R(R+1)/2).
* "Decode Token Parallelism: Memory-Efficient Distributed Attention Parallelism
  for Scalable LLM Decoding" -- §4.3 (decode step order: rotary embedding,
  append K/V, attention; then output projection, residual and normalization,
  MLP), Eq. 4 (fp32 log-sum-exp partials).
* The paper-daily.com summary of ConfluxServe -- the worked waterfill example
  (decode loads 40/10/10/0, cap 300, capacities 260/290/290/300, budget 1140).

Modules:

* ``numerics``  -- exact decoding of stored values and RNE rounding to storage.
* ``layer``     -- the layer, row by row in fp64 (pinned: brute force, library
  Llama layer, closed forms, invariants).
* ``brute``     -- pure-Python loops for tiny inputs (a second formulation used
  only to pin ``layer``).
* ``waterfill`` -- latency model (Eq. 2-11) and waterfill dispatch
  (Algorithm 2) in Python integers and doubles (pinned: the worked example,
  brute-force min-max enumeration, linear scan of levels, closed forms).
* ``estimator`` -- fitting the latency model's base functions (App. D) and the
  contention factors of Eq. 4 from profiles (pinned: exact recovery from noiseless
  data, closed forms, optimality of the relative-error loss).
* ``scheduler`` -- SLO-aware scheduler (Algorithm 1), dual-mode decode
  placement (Algorithm 3) and Moore-Hodgson admission (Algorithm 4) (pinned:
  brute-force largest on-time set, hand-worked cases, invariants).

Parity status: every function here has at least one pin in
``tests/test_oracle_*.py``; none is "parity unpinned".
"""
