// probe.hip -- read-only HBM probe: the bandwidth ceiling the attention
// kernels are measured against on the same device.
//
// The decode step is bound by reading the KV cache ("9 Decode and KV Cache",
// section 9.8: bytes moved over elapsed time, against the bandwidth the
// memory sustains; SoK paper section 1.1). Besides the vendor peak, a kernel
// is compared with what plain loads of the same shape achieve here:
//  - sequential: `waves` waves read a contiguous buffer, each wave taking
//    4 KiB per step (one 16-byte load per lane, four per step) in a
//    grid-stride walk;
//  - tiles: each wave reads its share of a list of tiles (whole tiles of
//    `tile_bytes` at given byte offsets, for example the (block, head) K and
//    V tiles of a paged cache in the order the attention kernel visits them),
//    with kTileDepth tiles in flight.
// Both use the attention kernel's non-temporal 16-byte loads, and every dword
// loaded is folded into a per-lane checksum written to `sink`, so no load can
// be dropped or narrowed by the compiler.
#include "device_common.h"
#include "pda_internal.h"


namespace pda {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kTileDepth = 4;   // tiles in flight per wave (two 8 KiB K + V blocks)
constexpr int kOffChunk = 512;  // tile offsets staged in LDS per wave at a time

__device__ __forceinline__ u32x4 ld_nt(const char* p) {
    return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return (v.x ^ v.y) ^ (v.z ^ v.w); }

__global__ void __launch_bounds__(kProbeThreads) k_probe_seq(const char* buf, int64_t steps,
                                                             int32_t waves, uint32_t* sink) {
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
    uint32_t acc = 0;
    // step s of wave w: bytes [(s * waves + w) * 4096, +4096)
    for (int64_t s = 0; s < steps; ++s) {
        const char* p = buf + ((s * waves + w) << 12) + 16 * lane;
        const u32x4 a = ld_nt(p), b = ld_nt(p + 1024), c = ld_nt(p + 2048), d = ld_nt(p + 3072);
        acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
    }
    sink[(int64_t)w * 64 + lane] = acc;
}

template <int LOADS>
__global__ void __launch_bounds__(kProbeThreads) k_probe_tiles(const char* buf,
                                                               const int64_t* off,
                                                               int64_t n_tiles, int32_t waves,
                                                               uint32_t* sink) {
    constexpr int D = kTileDepth;
    // Tile offsets pass through LDS in chunks of kOffChunk per wave: the
    // issuer's LDS reads are waited on by their own counter, so a tile's wait
    // drains that tile's loads only.
    __shared__ int64_t off_lds[kProbeThreads / 64][kOffChunk];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int w = blockIdx.x * (kProbeThreads / 64) + wv;
    const int64_t t0 = (int64_t)w * n_tiles / waves, t1 = (int64_t)(w + 1) * n_tiles / waves;
    int64_t* so = off_lds[wv];
    uint32_t acc = 0;
    u32x4 r[D][LOADS];
    auto issue = [&](int slot, int i) {
        const char* p = buf + so[i] + 16 * lane;
#pragma unroll
        for (int l = 0; l < LOADS; ++l) r[slot][l] = ld_nt(p + 1024 * l);
    };
    auto consume = [&](int slot) {
#pragma unroll
        for (int l = 0; l < LOADS; ++l) acc ^= fold(r[slot][l]);
    };
    for (int64_t c0 = t0; c0 < t1; c0 += kOffChunk) {
        const int n = (int)min((int64_t)kOffChunk, t1 - c0);
        for (int k = lane; k < n; k += 64) so[k] = off[c0 + k];
        __builtin_amdgcn_s_waitcnt(0);   // the chunk's offsets are in LDS
        __builtin_amdgcn_wave_barrier();
        // steady state without conditions (as in the attention kernel), so
        // the wait before each tile drains only that tile's loads
        int i = 0;
        if (n >= 2 * D) {
#pragma unroll
            for (int s = 0; s < D; ++s) {
                issue(s, s);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (; i + 2 * D <= n; i += D) {
#pragma unroll
                for (int s = 0; s < D; ++s) {
                    consume(s);
                    issue(s, i + s + D);
                    // keep each slot's refill in place, so the loads stay in
                    // slot order
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < D; ++s)
                if (s < n) issue(s, s);
        }
#pragma unroll
        for (int k = 0; k < 2 * D; ++k) {
            if (i + k < n) {
                consume(k % D);
                if (i + k + D < n) issue(k % D, i + k + D);
            }
        }
        __builtin_amdgcn_wave_barrier();   // every lane is done with this chunk's offsets
    }
    sink[(int64_t)w * 64 + lane] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, const int64_t* tile_offsets,
                             int64_t n_tiles, int32_t tile_bytes, int32_t waves,
                             uint32_t* sink, hipStream_t s) {
    const dim3 grid((unsigned)(waves / 4)), block(kProbeThreads);
    if (tile_offsets == nullptr) {
        const int64_t steps = (int64_t)(bytes / 4096) / waves;
        hipLaunchKernelGGL(k_probe_seq, grid, block, 0, s, (const char*)buf, steps, waves, sink);
    } else {
        switch (tile_bytes) {
            case 1024: hipLaunchKernelGGL((k_probe_tiles<1>), grid, block, 0, s,
                                          (const char*)buf, tile_offsets, n_tiles, waves, sink);
                       break;
            case 2048: hipLaunchKernelGGL((k_probe_tiles<2>), grid, block, 0, s,
                                          (const char*)buf, tile_offsets, n_tiles, waves, sink);
                       break;
            case 4096: hipLaunchKernelGGL((k_probe_tiles<4>), grid, block, 0, s,
                                          (const char*)buf, tile_offsets, n_tiles, waves, sink);
                       break;
            default:   hipLaunchKernelGGL((k_probe_tiles<8>), grid, block, 0, s,
                                          (const char*)buf, tile_offsets, n_tiles, waves, sink);
                       break;
        }
    }
    return hipGetLastError();
}

}  // namespace pda
