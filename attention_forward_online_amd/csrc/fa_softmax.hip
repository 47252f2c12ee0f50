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
// Two kernels:
//   fused   one chunk holds the whole row (one wave or one workgroup per row):
//           the exponentials stay in registers, so X is read once and Y
//           written once.
//   wide    rows wider than a chunk, one workgroup per (row, chunk) and pass:
//           pass 1 writes the chunk's (m, l) to the workspace; pass 2 merges
//           the row's chunk pairs in a fixed order, re-reads the chunk and
//           writes y = exp(x - m) / l (chunk 0 writes lse).
// The host walks the rows in blocks; launch k runs pass 2 of block k - 1 and
// pass 1 of block k, so pass 2 re-reads X from the memory-side Infinity Cache
// instead of HBM and the new reads overlap it.
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
// Rows up to this many bytes per block: a launch reads one block for pass 1
// and re-reads the previous block for pass 2, so two blocks of X should fit
// the 256 MB Infinity Cache next to the Y writes in flight.  Smaller blocks
// lose more to the gaps between launches (about 3 us each) than they gain.
constexpr long long kBlockBytes = 64LL << 20;
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
    // entries k0 + e outside [lo, hi) become -inf
    static __device__ __forceinline__ void mask_raw(u32x4_t &raw, int k0, int lo, int hi) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            if (k0 + w < lo || k0 + w >= hi) raw[w] = 0xff800000u;
    }
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
    static __device__ __forceinline__ void mask_raw(u32x4_t &raw, int k0, int lo, int hi) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t b = raw[w];
            if (k0 + 2 * w < lo || k0 + 2 * w >= hi) b = (b & 0xffff0000u) | 0xff80u;
            if (k0 + 2 * w + 1 < lo || k0 + 2 * w + 1 >= hi) b = (b & 0xffffu) | 0xff800000u;
            raw[w] = b;
        }
    }
};

// (m, l): max of the entries seen and sum of exp(x - m) over them; (-inf, 0)
// when every entry is masked.
struct ML {
    float m, l;
};

// No FMA contraction here: both products are rounded and then added, so
// merge(a, b) and merge(b, a) give the same bits (fp addition commutes) in
// every kernel that inlines it.
__device__ __forceinline__ ML merge(ML a, ML b) {
#pragma clang fp contract(off)
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
    unsigned *ticket;       // one-pass wide rows: the next (row, chunk) to hand out
    long long row0, row_end;          // fused kernels: rows [row0, row_end)
    long long norm_row0, norm_rows;   // wide rows: pass 2 over these rows ...
    long long stats_row0, stats_rows; // ... and pass 1 over these, in one launch
    long long cols;
    long long total_bytes;  // rows * cols * sizeof(T)
    int S;                  // chunks per row
    int spin_limit;         // one-pass wait: polls before the fallback
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
        const long long cap = (long long)(C * sizeof(T));
        load_bytes = (uint32_t)(avail < 0 ? 0 : (avail > cap ? cap : avail));
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
                                           float (&x)[C / TPR]) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int NV = C / (TPR * VN);
    if (g.load_bytes == 0) {   // chunk past the row's end (or cols == 0): touch nothing
#pragma unroll
        for (int e = 0; e < NV * VN; ++e) x[e] = neg_inf();
        return;
    }
    const rsrc_t rs = make_rsrc(p.X + g.start * (long long)sizeof(T), g.load_bytes);
    u32x4_t raw[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        raw[i] = load16<AUX>(rs, (uint32_t)((i * TPR + t) * VN * (int)sizeof(T)));
#pragma unroll
    for (int i = 0; i < NV; ++i) Elem<T>::widen(raw[i], &x[i * VN]);
    if (!g.interior) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                const int k = (i * TPR + t) * VN + e;
                if (k < g.lo || k >= g.hi) x[i * VN + e] = neg_inf();
            }
    }
}

// Store the VN values y of the vector at chunk element k0: one 16-byte store
// when the vector lies inside the row, element by element where it straddles
// the row edge.
template <typename T, int C>
__device__ __forceinline__ void store_vec(T *yc, const ChunkGeom<T, C> &g, int k0, const float *y) {
    constexpr int VN = Elem<T>::kVec;
    if (g.interior || (k0 >= g.lo && k0 + VN <= g.hi)) {
        __builtin_nontemporal_store(Elem<T>::narrow(y), reinterpret_cast<u32x4_t *>(yc + k0));
    } else {
#pragma unroll
        for (int e = 0; e < VN; ++e)
            if (k0 + e >= g.lo && k0 + e < g.hi) Elem<T>::store1(yc + k0 + e, y[e]);
    }
}

// Store y for this thread's elements of the chunk.
template <typename T, int TPR, int C>
__device__ __forceinline__ void store_chunk(const Params &p, const ChunkGeom<T, C> &g, int t,
                                            const float (&y)[C / TPR]) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int NV = C / (TPR * VN);
    T *yc = reinterpret_cast<T *>(p.Y) + g.start;
#pragma unroll
    for (int i = 0; i < NV; ++i) store_vec<T, C>(yc, g, (i * TPR + t) * VN, &y[i * VN]);
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
__device__ __forceinline__ void stats_item(const Params &p, long long r, int c, ML *sh) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int C = kThreads * Elem<T>::kNV * VN;
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
__device__ __forceinline__ void norm_item(const Params &p, long long r, int c, ML *sh) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int C = kThreads * Elem<T>::kNV * VN;
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

// One launch of the wide-row pipeline: the first norm_rows * grid_chunks
// workgroups run pass 2 over rows [norm_row0, +norm_rows) (whose pairs an
// earlier launch wrote), the rest run pass 1 over rows [stats_row0,
// +stats_rows).  The two ranges are disjoint, so no workgroup waits for
// another; pass 1 of the next block of rows streams from HBM while pass 2
// re-reads the previous block from the Infinity Cache.
template <typename T>
__global__ __launch_bounds__(kThreads) void softmax_wide_kernel(Params p) {
    __shared__ ML sh[kWaves];
    const long long b = blockIdx.x;
    const long long n_norm = p.norm_rows * p.grid_chunks;
    if (b < n_norm) {
        norm_item<T>(p, p.norm_row0 + b / p.grid_chunks, (int)(b % p.grid_chunks), sh);
    } else {
        const long long u = b - n_norm;
        stats_item<T>(p, p.stats_row0 + u / p.S, (int)(u % p.S), sh);
    }
}

// One-pass wide rows.  The 64-bit pair (m, l) of a chunk is published with
// one device-scope atomic store; l = -1 (never a real sum) marks "not yet".
// At most this many chunks per row on the one-pass path (2 Mi fp32 or 4 Mi
// bf16 elements): the chip must hold one row's workgroups at once.
constexpr int kCoopMaxChunks = 128;
// Vectors per thread in a one-pass chunk: 64 KiB per workgroup for either
// element type (fewer, larger chunks mean fewer tickets and shorter waits).
template <typename T> constexpr int coop_nv() { return 64 * 1024 / (kThreads * 16); }
template <typename T> constexpr int coop_chunk() { return kThreads * coop_nv<T>() * Elem<T>::kVec; }
constexpr int kSpinLimit = 1 << 16;        // polls before the fallback (about 0.1 s)
// Polls of the next one-pass launches; only the test hook changes it.
int g_spin_limit = kSpinLimit;
constexpr float kUnset = -1.f;

__device__ __forceinline__ uint64_t pack_ml(ML s) {
    return (uint64_t)__builtin_bit_cast(uint32_t, s.m) |
           ((uint64_t)__builtin_bit_cast(uint32_t, s.l) << 32);
}
__device__ __forceinline__ ML unpack_ml(uint64_t v) {
    return {__builtin_bit_cast(float, (uint32_t)v), __builtin_bit_cast(float, (uint32_t)(v >> 32))};
}

__global__ __launch_bounds__(kThreads) void softmax_reset_kernel(unsigned *ticket, f32x2_t *pairs,
                                                                 long long n) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i == 0) *ticket = 0u;
    if (i < n) pairs[i] = f32x2_t{neg_inf(), kUnset};
}

// (m, l) of row r streamed by one workgroup, one 16-byte vector per thread at
// a time (the bounded wait's fallback; X is never written on this path),
// bit for bit the pair the waiting path merges.
template <typename T>
__device__ ML stream_row_stats(const Params &p, long long r, ML *sh) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int C = coop_chunk<T>();
    constexpr int NV = coop_nv<T>();
    const int t = threadIdx.x;
    // every chunk's pair formed exactly as the workgroup that owns the chunk
    // forms it (same elements per thread, max first, then the exponentials
    // summed in the same order, the same workgroup merge), one vector in
    // registers at a time; thread j keeps the pair of chunk j
    ML mine{neg_inf(), 0.f};
#pragma unroll 1
    for (int j = 0; j < p.S; ++j) {
        const ChunkGeom<T, C> g(p, r, j);
        const rsrc_t rs = make_rsrc(p.X + g.start * (long long)sizeof(T), g.load_bytes);
        auto vec = [&](int i, float *x) {
            u32x4_t raw = g.load_bytes == 0
                ? u32x4_t{0u, 0u, 0u, 0u}
                : load16<0>(rs, (uint32_t)((i * kThreads + t) * VN * (int)sizeof(T)));
            if (!g.interior) Elem<T>::mask_raw(raw, (i * kThreads + t) * VN, g.lo, g.hi);
            Elem<T>::widen(raw, x);
        };
        float m = neg_inf();
#pragma unroll 1
        for (int i = 0; i < NV; ++i) {
            float x[VN];
            vec(i, x);
#pragma unroll
            for (int e = 0; e < VN; ++e) m = fmaxf(m, x[e]);
        }
        const float ms = m == neg_inf() ? 0.f : m;
        float l = 0.f;
#pragma unroll 1
        for (int i = 0; i < NV; ++i) {
            float x[VN];
            vec(i, x);
#pragma unroll
            for (int e = 0; e < VN; ++e) l += exp2_hw((x[e] - ms) * kLog2e);
        }
        const ML pair = group_merge<kThreads>(ML{m, l}, sh);
        __syncthreads();    // sh is written again for the next chunk
        if (t == j) mine = pair;
    }
    // then the row's pairs merge exactly as on the path that read them
    return group_merge<kThreads>(mine, sh);
}

// Wide rows in one pass over X: a workgroup takes the next (row, chunk)
// ticket, keeps its chunk's exponentials in registers, publishes the chunk
// pair, waits until the row's S pairs are there, merges them in index order
// and writes y.  Tickets are handed out in the order workgroups start, so a
// workgroup holding a ticket is resident, and it only waits for chunks of its
// own row; every earlier row has all its chunks held by resident workgroups
// that do not wait on later tickets, so the wait ends whenever the chip holds
// one row's chunks at once (S <= 128 here, against 1280 resident workgroups
// at 5 per CU).  The wait is still bounded: past the poll limit the
// workgroup streams the row itself (the same pair to the bit), so every
// wave exits.  X must not alias Y on this path (the fallback re-reads X).
template <typename T>
__global__ __launch_bounds__(kThreads) void softmax_coop_kernel(Params p) {
    constexpr int VN = Elem<T>::kVec;
    constexpr int NV = coop_nv<T>();
    constexpr int C = coop_chunk<T>();
    __shared__ ML sh[kWaves];
    __shared__ unsigned tk;
    if (threadIdx.x == 0) tk = atomicAdd(p.ticket, 1u);
    __syncthreads();
    const long long r = p.norm_row0 + tk / (unsigned)p.S;
    const int c = (int)(tk % (unsigned)p.S);
    const ChunkGeom<T, C> g(p, r, c);
    const int t = threadIdx.x;

    // the chunk stays in registers as raw 16-byte vectors
    u32x4_t raw[NV];
    if (g.load_bytes == 0) {
#pragma unroll
        for (int i = 0; i < NV; ++i) raw[i] = u32x4_t{0u, 0u, 0u, 0u};
    } else {
        const rsrc_t rs = make_rsrc(p.X + g.start * (long long)sizeof(T), g.load_bytes);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            raw[i] = load16<kAuxNT>(rs, (uint32_t)((i * kThreads + t) * VN * (int)sizeof(T)));
    }
    // entries outside the row become -inf in the raw registers, once
    if (!g.interior) {
#pragma unroll
        for (int i = 0; i < NV; ++i) Elem<T>::mask_raw(raw[i], (i * kThreads + t) * VN, g.lo, g.hi);
    }
    // Each pass widens the raw vectors again; the empty asm makes the raw
    // registers opaque between passes, so the compiler keeps the raw data
    // live instead of every widened float (64 VGPRs, not 128 for bf16).
    auto opaque = [&]() {
#pragma unroll
        for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(raw[i]));
    };
    auto elems = [&](int i, float *x) { Elem<T>::widen(raw[i], x); };
    float m = neg_inf();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        float x[VN];
        elems(i, x);
#pragma unroll
        for (int e = 0; e < VN; ++e) m = fmaxf(m, x[e]);
    }
    const float ms = m == neg_inf() ? 0.f : m;
    float l = 0.f;
    opaque();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        float x[VN];
        elems(i, x);
#pragma unroll
        for (int e = 0; e < VN; ++e) l += exp2_hw((x[e] - ms) * kLog2e);
    }
    const ML chunk = group_merge<kThreads>(ML{m, l}, sh);
    uint64_t *slots = reinterpret_cast<uint64_t *>(p.ws) + r * p.S;
    if (threadIdx.x == 0)
        __hip_atomic_store(slots + c, pack_ml(chunk), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // wait for the row's S pairs: thread j < S keeps pair j of the last poll
    // (each pair is one 64-bit atomic: the sentinel or the whole pair)
    ML mine{neg_inf(), 0.f};
    bool ready = false;
    for (int it = 0; it < p.spin_limit; ++it) {
        int ok = 1;
        if ((int)threadIdx.x < p.S) {
            mine = unpack_ml(__hip_atomic_load(slots + threadIdx.x, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT));
            ok = mine.l != kUnset;
        }
        if (__syncthreads_and(ok)) {
            ready = true;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    const ML row = ready ? group_merge<kThreads>(mine, sh) : stream_row_stats<T>(p, r, sh);

    // y = exp(x - M) / L from the registers (as the two-pass norm pass does)
    const float inv = row.l > 0.f ? 1.f / row.l : 0.f;
    const float M = row.m == neg_inf() ? 0.f : row.m;
    T *yc = reinterpret_cast<T *>(p.Y) + g.start;
    opaque();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        float y[VN];
        Elem<T>::widen(raw[i], y);
#pragma unroll
        for (int e = 0; e < VN; ++e) y[e] = exp2_hw((y[e] - M) * kLog2e) * inv;
        store_vec<T, C>(yc, g, (i * kThreads + t) * VN, y);
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

// Workspace: a 16-byte header (the ticket counter), then the chunk pairs
// (sized for the two-pass chunks, which are never larger than one-pass ones).
constexpr size_t kWsHeader = 16;

template <typename T>
size_t workspace_bytes_t(long long rows, long long cols) {
    constexpr int VN = Elem<T>::kVec;
    const long long head = cols % VN == 0 ? 0 : VN - 1;
    if (cols + head <= chunk_elems<T>(kThreads)) return 0;
    return kWsHeader + (size_t)rows * (size_t)chunks_per_row<T>(cols) * sizeof(f32x2_t);
}

template <typename T>
hipError_t launch_softmax_t(const SoftmaxArgs &a, hipStream_t stream) {
    constexpr int VN = Elem<T>::kVec;
    Params p{};
    p.X = static_cast<const uint8_t *>(a.X);
    p.Y = static_cast<uint8_t *>(a.Y);
    p.LSE = a.LSE;
    p.spin_limit = g_spin_limit;
    p.ticket = static_cast<unsigned *>(a.workspace);
    p.ws = reinterpret_cast<f32x2_t *>(static_cast<uint8_t *>(a.workspace) + kWsHeader);
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
    auto launch = [&](long long n0, long long nn, int gc, long long s0, long long sn) {
        p.norm_row0 = n0;
        p.norm_rows = nn;
        p.grid_chunks = gc;
        p.stats_row0 = s0;
        p.stats_rows = sn;
        const long long blocks = nn * gc + sn * p.S;
        hipLaunchKernelGGL((softmax_wide_kernel<T>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, p);
        return hipGetLastError();
    };
    if (!p.Y) {
        // log-sum-exp only: nothing is re-read, so no blocks: pass 1 over
        // every row, then one merging workgroup per row
        const long long max_rows = 0x7fffffffLL / p.S;
        for (long long r0 = 0; r0 < a.rows; r0 += max_rows) {
            const long long n = a.rows - r0 < max_rows ? a.rows - r0 : max_rows;
            hipError_t e = launch(0, 0, 1, r0, n);
            if (e == hipSuccess) e = launch(r0, n, 1, 0, 0);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const long long s_coop = (a.cols + head + coop_chunk<T>() - 1) / coop_chunk<T>();
    if (s_coop <= kCoopMaxChunks && a.X != a.Y) {
        // one pass over X: reset the ticket and the pairs, then one
        // workgroup per (row, chunk) ticket
        p.S = (int)s_coop;
        const long long max_rows = 0x7fffffffLL / p.S;
        for (long long r0 = 0; r0 < a.rows; r0 += max_rows) {
            const long long n = a.rows - r0 < max_rows ? a.rows - r0 : max_rows;
            const long long npairs = n * p.S;
            hipLaunchKernelGGL(softmax_reset_kernel, dim3((unsigned)((npairs + kThreads - 1) / kThreads)),
                               dim3(kThreads), 0, stream, p.ticket, p.ws + r0 * p.S, npairs);
            p.norm_row0 = r0;
            hipLaunchKernelGGL((softmax_coop_kernel<T>), dim3((unsigned)npairs), dim3(kThreads), 0,
                               stream, p);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // in place, or rows of more than kCoopMaxChunks chunks: two passes over X
    const long long row_bytes = a.cols * (long long)sizeof(T);
    long long block = kBlockBytes / row_bytes;
    if (block < 1) block = 1;
    const long long max_block = 0x7fffffffLL / (2LL * p.S);
    if (block > max_block) block = max_block;
    // launch k: pass 2 of block k - 1 together with pass 1 of block k
    for (long long r0 = 0, prev0 = 0, prevn = 0;; ) {
        const long long n = a.rows - r0 < block ? a.rows - r0 : block;
        if (prevn == 0 && n == 0) break;
        const hipError_t e = launch(prev0, prevn, p.S, r0, n);
        if (e != hipSuccess) return e;
        prev0 = r0;
        prevn = n;
        r0 += n;
    }
    return hipSuccess;
}

}  // namespace

size_t softmax_workspace_bytes(long long rows, long long cols, bool is_bf16) {
    return is_bf16 ? workspace_bytes_t<uint16_t>(rows, cols) : workspace_bytes_t<float>(rows, cols);
}

void set_softmax_spin_limit(int limit) { g_spin_limit = limit < 0 ? kSpinLimit : limit; }

hipError_t launch_softmax(const SoftmaxArgs &a, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? launch_softmax_t<uint16_t>(a, stream) : launch_softmax_t<float>(a, stream);
}

}  // namespace fa
