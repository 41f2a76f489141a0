// Measurement kernels of the benchmark (libbsprobe.so): a plain streaming
// read of a buffer and an empty kernel.  They isolate the read ceiling and
// the dispatch floor that a GEMV's time is read against; nothing of the hot
// path runs here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bs_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Thread t of workgroup b reads the 16-byte chunks b*256*U + t + 256*u,
// u < U (a workgroup reads 4 KB contiguous per step), through a buffer
// resource bounded at `bytes`: chunks past the end read zero.
template <int U>
__global__ __launch_bounds__(256) void stream_read(const uint8_t *__restrict__ src,
                                                   uint32_t bytes, int64_t *__restrict__ sink) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(src), 0, (int)bytes, 0x00020000);
    const uint32_t base = (uint32_t)blockIdx.x * 256u * U * 16u + threadIdx.x * 16u;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + u * 4096u, 0, 2);
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Grid-stride form: a fixed grid of workgroups, each reading 32 KB
// contiguous per step (256 threads x 8 loads 4 KB apart) and striding by the
// whole grid's 32 KB blocks; for large buffers, where the one-pass form's
// grid grows with the bytes.  Offsets stay below 2^32: bytes < 2^31 and the
// stride is at most 2^31.
__global__ __launch_bounds__(256) void stream_read_strided(const uint8_t *__restrict__ src,
                                                           uint32_t bytes,
                                                           int64_t *__restrict__ sink) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(src), 0, (int)bytes, 0x00020000);
    const uint32_t stride = gridDim.x * 32768u;
    uint32_t acc = 0;
    for (uint32_t base = blockIdx.x * 32768u + threadIdx.x * 16u; base < bytes; base += stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + u * 4096u, 0, 2);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" int64_t bs_probe_read_sink_count(uint64_t bytes, int32_t per_thread) {
    if (bytes < 1 || bytes > (1ull << 31) - 16) return -3;   // offsets stay in 32 bits
    if (per_thread != 1 && per_thread != 2 && per_thread != 4 && per_thread != 8) return -3;
    const uint64_t per_block = 256ull * 16ull * (uint64_t)per_thread;
    return (int64_t)((bytes + per_block - 1) / per_block) * 256;
}

extern "C" int32_t bs_probe_read(const void *src, uint64_t bytes, int32_t per_thread,
                                 int64_t *sink, void *stream) {
    if (!src || !sink) return -1;
    const int64_t n = bs_probe_read_sink_count(bytes, per_thread);
    if (n < 0) return -3;
    if (((uintptr_t)src & 15) || ((uintptr_t)sink & 7)) return -3;
    const dim3 grid((unsigned)(n / 256));
    hipStream_t st = (hipStream_t)stream;
    const uint8_t *p = static_cast<const uint8_t *>(src);
    const uint32_t b = (uint32_t)bytes;
    switch (per_thread) {
    case 1: hipLaunchKernelGGL(stream_read<1>, grid, dim3(256), 0, st, p, b, sink); break;
    case 2: hipLaunchKernelGGL(stream_read<2>, grid, dim3(256), 0, st, p, b, sink); break;
    case 4: hipLaunchKernelGGL(stream_read<4>, grid, dim3(256), 0, st, p, b, sink); break;
    default: hipLaunchKernelGGL(stream_read<8>, grid, dim3(256), 0, st, p, b, sink); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int32_t bs_probe_read_strided(const void *src, uint64_t bytes, int32_t blocks,
                                         int64_t *sink, void *stream) {
    if (!src || !sink) return -1;
    if (bytes < 1 || bytes > (1ull << 31) - 16 || blocks < 1 || blocks > 65536) return -3;
    if (((uintptr_t)src & 15) || ((uintptr_t)sink & 7)) return -3;
    hipLaunchKernelGGL(stream_read_strided, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, static_cast<const uint8_t *>(src), (uint32_t)bytes,
                       sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int32_t bs_probe_empty(int32_t blocks, int32_t threads, void *stream) {
    if (blocks < 1 || blocks > (1 << 20) || threads < 64 || threads > 1024 || threads % 64)
        return -3;
    hipLaunchKernelGGL(empty_kernel, dim3((unsigned)blocks), dim3((unsigned)threads), 0,
                       (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
