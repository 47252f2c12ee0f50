// fa_softmax.hip -- streaming row softmax and log-sum-exp on gfx950.
//
// y = exp(x - max) / sum exp(x - max) and lse = max + ln sum exp(x - max) for
// every row of a [rows, cols] matrix, for rows of any width.  The statistics
// are the online-softmax pair (m, l): a running max and the denominator
// referred to it ('Online Softmax -- the mathematical heart of FlashAttention',
// section 4).  Two partial pairs over disjoint parts of a row combine with
// the associative merge m = max(m1, m2), l = exp(m1 - m) l1 + exp(m2 - m) l2
// ('Online Softmax & FlashAttention' (interview lesson), Step 1), so a row
// can be cut anywhere: every thread forms the pair of its own elements, the
// pairs merge across the wave and the workgroup, and rows wider than one
// workgroup's chunk merge the chunk pairs in a second kernel -- the streaming
// softmax for rows wider than on-chip memory that the 'Online Softmax'
// research-hub page ("Why it matters") names.
//
// Three kernels:
//   fused   one chunk holds the whole row (one wave or one workgroup per row):
//           the exponentials stay in registers, so X is read once and Y
//           written once.
//   stats   wide rows, one workgroup per (row, chunk): the chunk's (m, l)
//           goes to the workspace.
//   norm    wide rows, one workgroup per (row, chunk): merges the row's chunk
//           pairs in a fixed order, re-reads the chunk and writes
//           y = exp(x - m) / l; chunk 0 writes lse.
// The host runs stats and norm over blocks of rows small enough that the
// norm pass re-reads X from the memory-side Infinity Cache instead of HBM.
//
// Layout: X, Y row-major [rows, cols] (fp32 or bf16), 16-byte aligned base;
// rows need not be aligned.  Each chunk starts at a 16-byte boundary of the
// flat array (the row's first element rounded down); elements of a loaded
// vector outside the row are masked to -inf and never stored.  -inf inputs are
// masked entries; a row with no finite entry gives y = 0 and lse = -inf.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Rows up to this many bytes per block of stats + norm launches, so that most
// of the block's X is still in the 256 MB Infinity Cache when the norm pass
// reads it again (its Y writes compete for the same cache).  Smaller blocks
// lose more to the gaps between launches (about 3 us each) than they gain.
constexpr long long kBlockBytes = 128LL << 20;
// Cache policy bit for loads and stores that are the last touch (nt).
constexpr int kAuxNT = 2;

template <typename T> struct Elem;
// kVec: elements per 16-byte vector; kNV: vectors per thread per chunk, so
// every wide-row chunk holds 8192 elements (32 KiB fp32, 16 KiB bf16).
template <> struct Elem<float> {
    static constexpr int kVec = 4;
    static constexpr int kNV = 8;
    static __device__ __forceinline__ void widen(u32x4_t raw, float *x) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t b = raw[w];
            x[w] = __builtin_bit_cast(float, b);
        }
    }
    static __device__ __forceinline__ u32x4_t narrow(const float *y) {
        u32x4_t r;
#pragma unroll
        for (int w = 0; w < 4; ++w) r[w] = __builtin_bit_cast(uint32_t, y[w]);
        return r;
    }
    static __device__ __forceinline__ void store1(float *p, float y) { *p = y; }
};
template <> struct Elem<uint16_t> {
    static constexpr int kVec = 8;
    static constexpr int kNV = 4;
    static __device__ __forceinline__ void widen(u32x4_t raw, float *x) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t b = raw[w];
            x[2 * w] = __builtin_bit_cast(float, b << 16);
            x[2 * w + 1] = __builtin_bit_cast(float, b & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ u32x4_t narrow(const float *y) {
        u32x4_t r;
#pragma unroll
        for (int w = 0; w < 4; ++w) r[w] = pack_bf16x2(y[2 * w], y[2 * w + 1]);
        return r;
    }
    static __device__ __forceinline__ void store1(uint16_t *p, float y) {
        *p = (uint16_t)(pack_bf16x2(y, 0.f) & 0xffffu);
    }
};

// (m, l): max of the entries seen and sum of exp(x - m) over them; (-inf, 0)
// when every entry is masked.
struct ML {
    float m, l;
};

__device__ __forceinline__ ML merge(ML a, ML b) {
    const float m = fmaxf(a.m, b.m);
    const float ms = m == neg_inf() ? 0.f : m;   // two masked sides: exp(-inf) = 0, no NaN
    return {m, a.l * exp2_hw((a.m - ms) * kLog2e) + b.l * exp2_hw((b.m - ms) * kLog2e)};
}

// Butterfly over the 64 lanes.  merge is commutative in floating point, so
// partners compute identical values and every lane ends with the same pair.
__device__ __forceinline__ ML wave_merge(ML s) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        s = merge(s, ML{shfl_xor_f32(s.m, off), shfl_xor_f32(s.l, off)});
    return s;
}

// Pair of the whole group (one wave, or the 4 waves of the workgroup); the
// cross-wave merge runs in a fixed order, so every thread gets the same bits.
template <int TPR>
__device__ __forceinline__ ML group_merge(ML s, ML *sh) {
    s = wave_merge(s);
    if constexpr (TPR == 64) {
        return s;
    } else {
        static_assert(TPR == kThreads, "a group is one wave or the whole workgroup");
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) sh[wave] = s;
        __syncthreads();
        return merge(merge(sh[0], sh[1]), merge(sh[2], sh[3]));
    }
}

struct Params {
    const uint8_t *X;
    uint8_t *Y;             // nullptr: log-sum-exp only
    float *LSE;
    f32x2_t *ws;            // [rows][S] chunk pairs (wide rows)
    long long row0, row_end;
    long long cols;
    long long total_bytes;  // rows * cols * sizeof(T)
    int S;                  // chunks per row
    int grid_chunks;        // chunk slots per row in this grid (S, or 1 when only lse is written)
};

// Where chunk c of row r sits.  The chunk starts at the row's first element
// rounded down to a 16-byte boundary, plus c whole chunks; chunk elements k in
// [lo, hi) belong to the row.
template <typename T, int C>
struct ChunkGeom {
    long long start;        // flat element index of chunk element 0
    int lo, hi;
    uint32_t load_bytes;    // bytes the buffer resource covers (loads past it return 0)
    bool interior;

    __device__ __forceinline__ ChunkGeom(const Params &p, long long r, int c) {
        constexpr int VN = Elem<T>::kVec;
        const long long f0 = r * p.cols;
        const long long a0 = f0 & ~(long long)(VN - 1);
        start = a0 + (long long)c * C;
        const long long p0 = start - f0;   // row position of chunk element 0
        const long long lo64 = -p0, hi64 = p.cols - p0;
        lo = (int)(lo64 < 0 ? 0 : (lo64 > C ? C : lo64));
        hi = (int)(hi64 < 0 ? 0 : (hi64 > C ? C : hi64));
        interior = lo == 0 && hi == C;
        // cover the row's part of the chunk, rounded up to whole 16-byte
        // vectors (a partial last vector never crosses a page: the base is
        // 16-byte aligned), and never past the end of the matrix rounded up
        const long long row_end16 = ((f0 + p.cols) * (long long)sizeof(T) + 15) & ~15LL;
        const long long mat_end16 = (p.total_bytes + 15) & ~15LL;
        long long avail = (row_end16 < mat_end16 ? row_end16 : mat_end16) - start * (long long)sizeof(T);
        if (hi <= lo) avail = 0;
        load_bytes = (uint32_t)(avail < 0 ? 0 : (avail > (long long)C * sizeof(T) ? (long long)C * sizeof(T) : avail));
    }
};

template <int AUX>
__device__ __forceinline__ u32x4_t load16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}

// Load this thread's NV vectors of the chunk and widen them to fp32, with
// elements outside the row set to -inf.
template <typename T, int TPR, int C, int AUX>
__device__ __forceinline__ void load_chunk(const Params &p, const ChunkGeom<T, C> &g, int t,
                                           float (&x)[Elem<T>::kNV * Elem<T>::kVec]) {
    constexpr int VN = Elem<T>::kVec;
    if (g.load_bytes == 0) {   // chunk past the row's end (or cols == 0): touch nothing
#pragma unroll
        for (int e = 0; e < Elem<T>::kNV * VN; ++e) x[e] = neg_inf();
        return;
    }
    const rsrc_t rs = make_rsrc(p.X + g.start * (long long)sizeof(T), g.load_bytes);
    u32x4_t raw[Elem<T>::kNV];
#pragma unroll
    for (int i = 0; i < Elem<T>::kNV; ++i)
        raw[i] = load16<AUX>(rs, (uint32_t)((i * TPR + t) * VN * (int)sizeof(T)));
#pragma unroll
    for (int i = 0; i < Elem<T>::kNV; ++i) Elem<T>::widen(raw[i], &x[i * VN]);
    if (!g.interior) {
#pragma unroll
        for (int i = 0; i < Elem<T>::kNV; ++i)
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                const int k = (i * TPR + t) * VN + e;
                if (k < g.lo || k >= g.hi) x[i * VN + e] = neg_inf();
            }
    }
}

// Store y for this thread's elements of the chunk: whole 16-byte vectors in
// the interior, element by element where the vector straddles the row edge.
template <typename T, int TPR, int C>
__device__ __forceinline__ void store_chunk(const Params &p, const ChunkGeom<T, C> &g, int t,
                                            const float (&y)[Elem<T>::kNV * Elem<T>::kVec]) {
    constexpr int VN = Elem<T>::kVec;
    T *yc = reinterpret_cast<T *>(p.Y) + g.start;
#pragma unroll
    for (int i = 0; i < Elem<T>::kNV; ++i) {
        const int k0 = (i * TPR + t) * VN;
        if (g.interior || (k0 >= g.lo && k0 + VN <= g.hi)) {
            __builtin_nontemporal_store(Elem<T>::narrow(&y[i * VN]),
                                        reinterpret_cast<u32x4_t *>(yc + k0));
        } else {
#pragma unroll
            for (int e = 0; e < VN; ++e)
                if (k0 + e >= g.lo && k0 + e < g.hi) Elem<T>::store1(yc + k0 + e, y[i * VN + e]);
        }
    }
}

__device__ __forceinline__ float lse_of(ML s) {
    return s.l > 0.f ? s.m + log2_hw(s.l) * kLn2 : neg_inf();
}

// One chunk = the whole row: a wave (TPR 64) or the workgroup (TPR 256).
template <typename T, int TPR>
__global__ __launch_bounds__(kThreads) void softmax_fused_kernel(Params p) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int C = TPR * Elem<T>::kNV * VN;
    __shared__ ML sh[kWaves];
    const int t = threadIdx.x % TPR;
    const long long r = p.row0 + (long long)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
    if (r >= p.row_end) return;   // group-uniform; only whole waves leave (TPR 64)

    const ChunkGeom<T, C> g(p, r, 0);
    float x[Elem<T>::kNV * VN];
    load_chunk<T, TPR, C, kAuxNT>(p, g, t, x);
    float m = neg_inf();
#pragma unroll
    for (int e = 0; e < Elem<T>::kNV * VN; ++e) m = fmaxf(m, x[e]);
    const float ms = m == neg_inf() ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < Elem<T>::kNV * VN; ++e) {
        x[e] = exp2_hw((x[e] - ms) * kLog2e);
        l += x[e];
    }
    const ML row = group_merge<TPR>(ML{m, l}, sh);
    if (p.Y) {
        // y = exp(x - ms) * exp(ms - M) / L; a thread with no visible entry
        // holds zeros and takes factor 0 (exp(ms - M) could overflow there)
        const float inv = row.l > 0.f ? 1.f / row.l : 0.f;
        const float f = m == neg_inf() ? 0.f : exp2_hw((ms - row.m) * kLog2e) * inv;
#pragma unroll
        for (int e = 0; e < Elem<T>::kNV * VN; ++e) x[e] *= f;
        store_chunk<T, TPR, C>(p, g, t, x);
    }
    if (t == 0) p.LSE[r] = lse_of(row);
}

// Wide rows, pass 1: (m, l) of chunk c of row r into the workspace.
template <typename T>
__global__ __launch_bounds__(kThreads) void softmax_stats_kernel(Params p) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int C = kThreads * Elem<T>::kNV * VN;
    __shared__ ML sh[kWaves];
    const long long r = p.row0 + blockIdx.x / p.S;
    const int c = (int)(blockIdx.x % p.S);
    const ChunkGeom<T, C> g(p, r, c);
    float x[Elem<T>::kNV * VN];
    // ordinary loads: the norm pass reads these bytes again soon
    load_chunk<T, kThreads, C, 0>(p, g, threadIdx.x, x);
    float m = neg_inf();
#pragma unroll
    for (int e = 0; e < Elem<T>::kNV * VN; ++e) m = fmaxf(m, x[e]);
    const float ms = m == neg_inf() ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < Elem<T>::kNV * VN; ++e) l += exp2_hw((x[e] - ms) * kLog2e);
    const ML s = group_merge<kThreads>(ML{m, l}, sh);
    if (threadIdx.x == 0) p.ws[r * p.S + c] = f32x2_t{s.m, s.l};
}

// Wide rows, pass 2: merge the row's chunk pairs, then y for chunk c.
template <typename T>
__global__ __launch_bounds__(kThreads) void softmax_norm_kernel(Params p) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int C = kThreads * Elem<T>::kNV * VN;
    __shared__ ML sh[kWaves];
    const long long r = p.row0 + blockIdx.x / p.grid_chunks;
    const int c = (int)(blockIdx.x % p.grid_chunks);
    const ChunkGeom<T, C> g(p, r, c);
    float x[Elem<T>::kNV * VN];
    if (p.Y) load_chunk<T, kThreads, C, kAuxNT>(p, g, threadIdx.x, x);
    // this thread's chunks j = t, t + 256, ... in order, then the group merge
    ML s{neg_inf(), 0.f};
    for (int j = threadIdx.x; j < p.S; j += kThreads) {
        const f32x2_t w = p.ws[r * p.S + j];
        s = merge(s, ML{w[0], w[1]});
    }
    const ML row = group_merge<kThreads>(s, sh);
    if (p.Y) {
        const float inv = row.l > 0.f ? 1.f / row.l : 0.f;
        const float M = row.m == neg_inf() ? 0.f : row.m;
#pragma unroll
        for (int e = 0; e < Elem<T>::kNV * VN; ++e) x[e] = exp2_hw((x[e] - M) * kLog2e) * inv;
        store_chunk<T, kThreads, C>(p, g, threadIdx.x, x);
    }
    if (c == 0 && threadIdx.x == 0) p.LSE[r] = lse_of(row);
}

template <typename T>
constexpr int chunk_elems(int tpr) { return tpr * Elem<T>::kNV * Elem<T>::kVec; }

// Chunks per row for the widest head offset the rows can have (0 when every
// row starts on a 16-byte boundary).
template <typename T>
long long chunks_per_row(long long cols) {
    constexpr int VN = Elem<T>::kVec;
    const long long head = cols % VN == 0 ? 0 : VN - 1;
    const long long C = chunk_elems<T>(kThreads);
    return (cols + head + C - 1) / C;
}

template <typename T>
size_t workspace_bytes_t(long long rows, long long cols) {
    constexpr int VN = Elem<T>::kVec;
    const long long head = cols % VN == 0 ? 0 : VN - 1;
    if (cols + head <= chunk_elems<T>(kThreads)) return 0;
    return (size_t)rows * (size_t)chunks_per_row<T>(cols) * sizeof(f32x2_t);
}

template <typename T>
hipError_t launch_softmax_t(const SoftmaxArgs &a, hipStream_t stream) {
    constexpr int VN = Elem<T>::kVec;
    Params p{};
    p.X = static_cast<const uint8_t *>(a.X);
    p.Y = static_cast<uint8_t *>(a.Y);
    p.LSE = a.LSE;
    p.ws = static_cast<f32x2_t *>(a.workspace);
    p.cols = a.cols;
    p.total_bytes = a.rows * a.cols * (long long)sizeof(T);
    const long long head = a.cols % VN == 0 ? 0 : VN - 1;
    if (a.cols + head <= chunk_elems<T>(64)) {
        // a wave per row, four rows per workgroup
        p.row0 = 0;
        p.row_end = a.rows;
        p.S = 1;
        p.grid_chunks = 1;
        const long long blocks = (a.rows + kWaves - 1) / kWaves;
        hipLaunchKernelGGL((softmax_fused_kernel<T, 64>), dim3((unsigned)blocks), dim3(kThreads),
                           0, stream, p);
        return hipGetLastError();
    }
    if (a.cols + head <= chunk_elems<T>(kThreads)) {
        p.row0 = 0;
        p.row_end = a.rows;
        p.S = 1;
        p.grid_chunks = 1;
        hipLaunchKernelGGL((softmax_fused_kernel<T, kThreads>), dim3((unsigned)a.rows),
                           dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
    p.S = (int)chunks_per_row<T>(a.cols);
    const long long row_bytes = a.cols * (long long)sizeof(T);
    // blocks only pay when the norm pass re-reads X, i.e. when Y is written
    long long block = p.Y ? kBlockBytes / row_bytes : a.rows;
    if (block < 1) block = 1;
    const long long max_block = 0x7fffffffLL / p.S;
    if (block > max_block) block = max_block;
    for (long long r0 = 0; r0 < a.rows; r0 += block) {
        p.row0 = r0;
        p.row_end = r0 + block < a.rows ? r0 + block : a.rows;
        const long long nr = p.row_end - r0;
        p.grid_chunks = p.S;
        hipLaunchKernelGGL((softmax_stats_kernel<T>), dim3((unsigned)(nr * p.S)), dim3(kThreads),
                           0, stream, p);
        p.grid_chunks = p.Y ? p.S : 1;
        hipLaunchKernelGGL((softmax_norm_kernel<T>), dim3((unsigned)(nr * p.grid_chunks)),
                           dim3(kThreads), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

size_t softmax_workspace_bytes(long long rows, long long cols, bool is_bf16) {
    return is_bf16 ? workspace_bytes_t<uint16_t>(rows, cols) : workspace_bytes_t<float>(rows, cols);
}

hipError_t launch_softmax(const SoftmaxArgs &a, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? launch_softmax_t<uint16_t>(a, stream) : launch_softmax_t<float>(a, stream);
}

}  // namespace fa
