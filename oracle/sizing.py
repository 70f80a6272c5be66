"""KV-cache byte accounting (TEST INFRASTRUCTURE, oracle).

Closed form ([SMTS] "Quantifying the KV-Cache Memory Wall"; [MTKV] "The
Anatomy of the KV-Cache Memory Wall"; [LLMI] "5. Mathematics: Sizing the KV
Cache"): the K and V caches of L layers, n_kv heads of width d, S tokens and
B sequences at p bytes per element occupy 2 * L * n_kv * d * S * B * p bytes.

The capacity model is the one [LLMI] "6. Implementation: KV Cache Memory &
Serving Simulator in TypeScript" describes, restated: weights take
params * 1e9 * p bytes (reported in binary GB rounded to 2 decimals); the KV
pool is what remains of the cluster's memory after weights and a per-GPU
activation overhead; a contiguous allocator reserves max_ctx tokens per
stream, a paged one only the average context. Its printed run (section
"Simulation Execution Output & State Transitions") pins the closed form.
"""

import math


def kv_bytes(L, n_kv, d, p, S=1, B=1):
    return 2 * L * n_kv * d * S * B * p


def kv_bytes_per_token(L, n_kv, d, p):
    return kv_bytes(L, n_kv, d, p)


def capacity(params_billion, L, n_kv, d, p, gpu_count, vram_per_gpu_gb,
             overhead_per_gpu_gb, avg_ctx, max_ctx):
    gib = 1024 ** 3
    per_token = kv_bytes_per_token(L, n_kv, d, p)
    weights_gb = round(params_billion * 1e9 * p / gib * 100) / 100
    usable_gb = max(0.0, gpu_count * vram_per_gpu_gb - weights_gb
                    - gpu_count * overhead_per_gpu_gb)
    usable_bytes = usable_gb * gib
    contiguous = math.floor(usable_bytes / (max_ctx * per_token))
    paged = math.floor(usable_bytes / (avg_ctx * per_token))
    gain = round((paged - contiguous) / contiguous * 100) if contiguous else 0
    return {
        "bytes_per_token": per_token,
        "weights_gb": weights_gb,
        "usable_gb": round(usable_gb * 10) / 10,
        "streams_contiguous": contiguous,
        "streams_paged": paged,
        "gain_percent": gain,
    }
