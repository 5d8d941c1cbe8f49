// Measurement reference: a plain streaming read of a device buffer, the
// "achievable" HBM bandwidth that the decode step's memory-bound kernels are
// compared against.  Not a step of the method.
//
// Each workgroup reads one contiguous chunk of the buffer; every lane keeps
// 8 non-temporal 16-byte loads in flight, and consecutive lanes read
// consecutive 16-byte pieces, so each load instruction of a wave covers 1 KB
// of contiguous memory and the workgroup 32 KB per round.  (Measured on
// MI355X over 2 GiB: 7.1-7.2 TB/s for any grid from 256 to 8192 workgroups,
// against 5.4-7.2 TB/s for a grid-stride layout.)  The pieces are folded
// into an XOR checksum so that no load can be dropped, and each wave adds its
// checksum to `sink` with one atomic XOR.
#include "bd_internal.h"
#include "bdiff_probe.h"

namespace bd {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                    size_t n16,
                                                                    uint32_t* __restrict__ sink) {
    constexpr size_t kRound = size_t(kProbeUnroll) * kProbeThreads;   // pieces per round
    const size_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = size_t(blockIdx.x) * chunk;
    const size_t end = beg + chunk < n16 ? beg + chunk : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t j = beg;
    for (; j < end && end - j >= kRound; j += kRound) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = __builtin_nontemporal_load(src + j + u * kProbeThreads + threadIdx.x);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    for (size_t t = j + threadIdx.x; t < end; t += kProbeThreads)
        acc ^= __builtin_nontemporal_load(src + t);
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0) atomicXor(sink, x);
}

}  // namespace
}  // namespace bd

extern "C" bd_status bd_probe_stream_read(const void* src, size_t n_bytes, int32_t grid,
                                          uint32_t* sink, hipStream_t stream) {
    if (!src || !sink) return BD_E_NULL;
    if (n_bytes == 0 || n_bytes % 16 != 0 || grid < 1 || grid > 65536) return BD_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return BD_E_ALIGN;
    hipLaunchKernelGGL(bd::stream_read_kernel, dim3(grid), dim3(bd::kProbeThreads), 0, stream,
                       static_cast<const bd::u32x4*>(src), n_bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? BD_OK : BD_E_LAUNCH;
}
