// Stream probe: a plain coalesced read of a device buffer, the reference
// kernel for achievable HBM read bandwidth ("a same-run reference kernel turns
// suspicion into proof": Part 2 post, "What we'd tell the next person").
// Every lane reads 16-byte units with U loads in flight, folds them with xor
// and writes one word, so no load can be elided.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef unsigned probe_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 probe_load(const uint4 *p, bool nt) {
    if (!nt) return *p;
    const probe_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const probe_u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// pattern 0: grid-stride rounds (all waves sweep one moving window);
// pattern 1: each wave streams its own contiguous range, as the matvec does;
// pattern 2: as 1, but each lane reads two adjacent 16-byte units;
// patterns 3, 4, 5: patterns 0, 1, 2 with non-temporal loads.
template <int U>
__global__ void __launch_bounds__(1024) stream_probe_kernel(const uint4 *buf, int64_t units, int pattern,
                                                            uint32_t *out) {
    const bool nt = pattern >= 3;
    if (pattern >= 3) pattern -= 3;
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t threads = int64_t(gridDim.x) * blockDim.x;
    uint32_t acc = 0;
    if (pattern == 0) {
        const int64_t rounds = (units + threads * U - 1) / (threads * U);
        for (int64_t r = 0; r < rounds; ++r) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = probe_load(buf + min((r * U + u) * threads + tid, units - 1), nt);
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    } else if (pattern == 2) {
        // each wave streams its own range; a lane reads two adjacent 16-byte
        // units per round (lane stride 32 bytes), U/2 such pairs in flight
        const int lane = threadIdx.x & 63;
        const int64_t waves = threads >> 6;
        const int64_t w = tid >> 6;
        const int64_t b = w * units / waves, e = (w + 1) * units / waves;
        const int64_t hi = e > b ? e - 1 : min(b, units - 1);
        const int64_t rounds = (e - b + 64 * U - 1) / (64 * U);
        for (int64_t r = 0; r < rounds; ++r) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = probe_load(buf + min(b + (r * U + (u & ~1)) * 64 + 2 * lane + (u & 1), hi), nt);
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    } else {
        const int lane = threadIdx.x & 63;
        const int64_t waves = threads >> 6;
        const int64_t w = tid >> 6;
        const int64_t b = w * units / waves, e = (w + 1) * units / waves;
        const int64_t hi = e > b ? e - 1 : min(b, units - 1);
        const int64_t rounds = (e - b + 64 * U - 1) / (64 * U);
        for (int64_t r = 0; r < rounds; ++r) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = probe_load(buf + min(b + (r * U + u) * 64 + lane, hi), nt);
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    out[tid] = acc;
}

}  // namespace qg
