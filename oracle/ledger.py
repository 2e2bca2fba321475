"""Model-state memory and communication ledger of ZeRO-DP (test infrastructure).

Closed forms as the pages state them, written out as plain functions:

* Paper translation "ZeRO：迈向训练万亿参数模型的内存优化技术", §3.1: mixed-
  precision Adam holds 2 bytes fp16 params + 2 bytes fp16 grads + K bytes of
  optimizer state per parameter, K = 12 (fp32 master, momentum, variance).
* Same page, §5.1-§5.3: per-device model states 4Ψ + KΨ/N_d (P_os),
  2Ψ + (K+2)Ψ/N_d (P_os+g), (4+K)Ψ/N_d (P_os+g+p).
* Same page, §7.1-§7.2: per-step data movement 2Ψ for DP, P_os and P_os+g,
  3Ψ for P_os+g+p.
* CMU 11-868 L18 notes, section on the memory and communication of the three
  stages: the same ledger with M bytes of optimizer state per parameter and K
  GPUs: DDP 4N+MN, ZeRO-1 4N+MN/K, ZeRO-2 2N+(2+M)N/K, ZeRO-3 (4+M)N/K.
"""

K_MIXED_ADAM = 12  # fp32 master + momentum + variance, bytes per parameter

STAGES = ("dp", "os", "os_g", "os_g_p")


def model_state_bytes(psi, n_d=1, stage="dp", k=K_MIXED_ADAM):
    """Bytes of model state on one data-parallel rank."""
    if stage == "dp":
        return (2 + 2 + k) * psi
    if stage == "os":
        return 4 * psi + k * psi / n_d
    if stage == "os_g":
        return 2 * psi + (k + 2) * psi / n_d
    if stage == "os_g_p":
        return (4 + k) * psi / n_d
    raise ValueError(stage)


def model_state_bytes_m(n_params, m_bytes, k_gpus, stage):
    """The CMU-notes form: M bytes of optimizer state per parameter, K GPUs."""
    n, m, k = n_params, m_bytes, k_gpus
    if stage == "ddp":
        return 4 * n + m * n
    if stage == "zero1":
        return 4 * n + m * n / k
    if stage == "zero2":
        return 2 * n + (2 + m) * n / k
    if stage == "zero3":
        return (4 + m) * n / k
    raise ValueError(stage)


def comm_volume_elems(psi, stage):
    """Elements sent and received per rank per training step."""
    if stage in ("dp", "os", "os_g"):
        return 2 * psi  # reduce-scatter + all-gather (= one all-reduce)
    if stage == "os_g_p":
        return 3 * psi  # + a parameter all-gather in forward and in backward
    raise ValueError(stage)
