// read_probe.hip - HBM read-rate probe used by the benchmark as context for
// the HBM-bound kernels' GB/s.  Not part of the attention path: it is built
// into its own library (libfa_probe.so) and nothing in libfa.so calls it.
//
// Reads a device buffer once with 16-byte non-temporal loads, the loads the
// paged kernels use, and writes nothing but (when a checksum takes one
// impossible value) a word of the sink, so its rate is the chip's practical
// read bandwidth for the access pattern:
//   * sequential: a grid-stride sweep over the buffer;
//   * 4 KiB chunks in a given random order: the grain of a paged KV cache
//     (one page of one head at d = 128 is 16 x 128 bf16 = 4 KiB).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                 // loads in flight per thread
constexpr int kSeqGroups = 16384;          // work groups of the sequential sweep
constexpr int kChunkWords = 4096 / 16;     // 16-byte words per 4 KiB chunk (one per thread)
constexpr int kChunksPerGroup = 32;
constexpr uint32_t kNever = 0x9e3779b9u;

__device__ __forceinline__ void keep(u32x4 acc, uint32_t* sink) {
    const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (r == kNever) sink[blockIdx.x & 255] = r;
}

__global__ __launch_bounds__(kThreads) void read_sequential(const u32x4* __restrict__ p, size_t n,
                                                            uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) x[j] = __builtin_nontemporal_load(p + i + j * stride);
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) acc ^= x[j];
    }
    for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    keep(acc, sink);
}

// work group b reads chunks order[b * kChunksPerGroup + c], c = 0 .. 31
__global__ __launch_bounds__(kThreads) void read_chunks(const u32x4* __restrict__ p,
                                                        const int32_t* __restrict__ order,
                                                        uint32_t* sink) {
    const int32_t* mine = order + (size_t)blockIdx.x * kChunksPerGroup;
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll 1
    for (int c = 0; c < kChunksPerGroup; c += kUnroll) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j)
            x[j] = __builtin_nontemporal_load(p + (size_t)mine[c + j] * kChunkWords + threadIdx.x);
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) acc ^= x[j];
    }
    keep(acc, sink);
}

}  // namespace

// buf: `bytes` of device memory (read); chunk_order: NULL for the sequential
// sweep, else bytes / 4096 int32 chunk indices, a permutation of 0 .. bytes /
// 4096 - 1 (read; bytes must then be a multiple of 128 KiB); sink: 1 KiB of
// device memory (written only in the impossible case).  Enqueued on `stream`
// (a hipStream_t, NULL = default), no synchronisation.  Returns a hipError_t.
extern "C" int fa_probe_read(const void* buf, size_t bytes, const int32_t* chunk_order,
                             void* sink, void* stream) {
    if (buf == nullptr || sink == nullptr || bytes < 16) return (int)hipErrorInvalidValue;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4* p = static_cast<const u32x4*>(buf);
    uint32_t* s = static_cast<uint32_t*>(sink);
    if (chunk_order == nullptr) {
        read_sequential<<<kSeqGroups, kThreads, 0, st>>>(p, bytes / 16, s);
    } else {
        const size_t group_bytes = (size_t)kChunksPerGroup * 4096;
        if (bytes % group_bytes != 0 || bytes / group_bytes > 2147483647u)
            return (int)hipErrorInvalidValue;
        read_chunks<<<(unsigned)(bytes / group_bytes), kThreads, 0, st>>>(p, chunk_order, s);
    }
    return (int)hipGetLastError();
}
