// fa_probe.hip -- measurement kernels that compute nothing of the attention
// path: the sustained rate of the matrix cores on a stream of independent bf16
// MFMAs, and the sustained HBM bandwidth of 16-byte loads (and stores).  Benchmarks
// put the attention kernels' rates next to what this GPU delivers for the bare
// operation each of them is bound by (the published peaks assume a clock the
// chip does not hold under sustained matrix-core load).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kProbeThreads = 256;

// Every wave issues `iters` rounds of eight 32x32x16 bf16 MFMAs on operands held
// in registers (no memory traffic inside the loop), into four independent
// accumulator chains, enough to keep the matrix pipe of its SIMD busy.  The
// operands are sixteen pseudo-random bf16 vectors per thread (random signs and
// mantissas, magnitudes in [0.5, 2)), a different pair for each MFMA of a round:
// the multipliers then toggle as they do on attention data (operands that never
// change draw less power, and the clock would settle higher than real data
// allows).  Each round adds the same products, so the sums grow linearly with
// `iters`; each thread writes the sum of its accumulators so that no product can
// be dropped.
constexpr int kMfmaPerRound = 8;

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(float *__restrict__ sink, int iters) {
    const int t = threadIdx.x;
    uint32_t h = ((uint32_t)blockIdx.x * kProbeThreads + (uint32_t)t) * 0x9e3779b9u + 0x7f4a7c15u;
    auto rnd = [&]() {   // xorshift32
        h ^= h << 13;
        h ^= h >> 17;
        h ^= h << 5;
        return h;
    };
    // two bf16 per word: sign, exponent 126 or 127 and the mantissa from the hash
    auto pair = [&]() { return (rnd() & 0x80ff80ffu) | 0x3f003f00u; };
    u32x4_t A[kMfmaPerRound], B[kMfmaPerRound];
#pragma unroll
    for (int j = 0; j < kMfmaPerRound; ++j) {
        A[j] = u32x4_t{pair(), pair(), pair(), pair()};
        B[j] = u32x4_t{pair(), pair(), pair(), pair()};
    }
    f32x16_t c[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kMfmaPerRound; ++j) c[j & 3] = mfma32(A[j], B[(j + 3) % kMfmaPerRound], c[j & 3]);
    }
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += (c[0][v] + c[1][v]) + (c[2][v] + c[3][v]);
    sink[(size_t)blockIdx.x * kProbeThreads + t] = s;
}

// Streaming read: the buffer is cut into chunks of kReadUnroll * 256
// consecutive 16-byte vectors (64 KiB) and each workgroup reads one contiguous
// run of them (consecutive workgroups, consecutive runs, as the decode's
// workgroups read their key ranges), thread t loading vectors t, t + 256, ...
// of a chunk, all kReadUnroll loads in flight and nontemporal (each byte is
// read once); the last, partial chunk goes by a grid-stride loop.  Each thread
// writes the XOR of the 32-bit words it read, so the XOR of all outputs is
// that of the buffer.
constexpr int kReadUnroll = 16;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t *__restrict__ src, size_t n16,
                                                                   uint32_t *__restrict__ sink) {
    constexpr size_t kChunk = (size_t)kProbeThreads * kReadUnroll;
    const size_t nch = n16 / kChunk;
    const size_t per = (nch + gridDim.x - 1) / gridDim.x;   // chunks per workgroup
    const size_t c0 = (size_t)blockIdx.x * per, c1 = c0 + per < nch ? c0 + per : nch;
    uint32_t x = 0;
    for (size_t ch = c0; ch < c1; ++ch) {
        const u32x4_t *p = src + ch * kChunk + threadIdx.x;
        u32x4_t v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + (size_t)u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (size_t i = nch * kChunk + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * kProbeThreads) {
        const u32x4_t v = __builtin_nontemporal_load(src + i);
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = x;
}

// Streaming copy: the read probe's chunking, each vector stored to the same
// offset of dst with a nontemporal store after all kReadUnroll loads of its
// chunk are in flight.
__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4_t *__restrict__ src,
                                                                   u32x4_t *__restrict__ dst, size_t n16) {
    constexpr size_t kChunk = (size_t)kProbeThreads * kReadUnroll;
    const size_t nch = n16 / kChunk;
    const size_t per = (nch + gridDim.x - 1) / gridDim.x;   // chunks per workgroup
    const size_t c0 = (size_t)blockIdx.x * per, c1 = c0 + per < nch ? c0 + per : nch;
    for (size_t ch = c0; ch < c1; ++ch) {
        const size_t i0 = ch * kChunk + threadIdx.x;
        u32x4_t v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i0 + (size_t)u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i0 + (size_t)u * kProbeThreads);
    }
    for (size_t i = nch * kChunk + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * kProbeThreads)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t launch_probe_mfma(float *sink, int blocks, int iters, hipStream_t stream) {
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream, sink, iters);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void *src, size_t bytes, uint32_t *sink, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4_t *>(src), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4_t *>(src), static_cast<u32x4_t *>(dst), bytes / 16);
    return hipGetLastError();
}

}  // namespace fa
