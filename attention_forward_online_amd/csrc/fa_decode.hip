// fa_decode.hip -- one-query split-KV decode (Flash-Decoding) on gfx950.
//
// With one query per sequence a split over queries leaves one block per head,
// far too little work for 256 compute units ('Online Softmax & FlashAttention'
// (interview lesson), Step 5).  The keys of each (b, h) are therefore cut into
// num_splits chunks; every chunk yields a partial state (m_c, l_c, o_c) and a
// second kernel merges the partials with the associative, commutative (m, l)
// merge of that page's Step 1, applied to o as well:
//     m = max(m1, m2);  l = e^(m1-m) l1 + e^(m2-m) l2;  o = e^(m1-m) o1 + e^(m2-m) o2
// with the reference m replaced by 0 when both sides are -inf.
//
// The split kernel is bound by the K/V stream from HBM, so it uses no matrix
// instruction.  K and V are read once, with nontemporal loads (they would only
// evict reusable lines from the caches), 16 rows of each in flight per lane
// (measured 6.83 TB/s, against 7.0 TB/s for a pure streaming read on the same
// 16 GiB).  Each lane owns 16 bytes of a key row (8 bf16 or 4 fp32), a key
// row is spread over LPR consecutive lanes whose partial dot products are
// summed by lane exchanges, and one wave-wide 16-byte load covers 64/LPR key
// rows.  Each group of LPR lanes keeps its own running (m, l, o) over the rows
// it reads (the recurrence of 'Online Softmax -- the mathematical heart of
// FlashAttention' section 5); the groups, then the four waves, are merged with
// the same (m, l) merge before the chunk's partial is written.
//
// Workspace layout (fp32): o[B][H][S][d], then m[B][H][S], then l[B][H][S];
// m is stored as scale*log2(e)*max score (-inf for an empty chunk).  The split
// kernel writes every record, empty chunks included, before the combine reads
// them, so the workspace needs no clearing between calls.
//
// For callers that cannot allocate, the library also holds one fixed scratch
// array per GPU (`scratch` below, kDecodeScratchBytes) that can stand in for
// the caller's workspace.
#include <mutex>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// Partial states of the decode entry point that allocates nothing.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code this name is only a handle: the device address comes from
// hipGetSymbolAddress (decode_scratch below).
__device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

// Device address of this GPU's `scratch`, looked up once per device (with that
// device current) and kept; a failed lookup is returned and retried next call.
hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void *addr[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 16;   // key-row loads of K (and of V) per lane in flight per iteration

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {   // bf16
    static constexpr int kPerLane = 8;
    __device__ static void widen(const u32x4_t &raw, float *f) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            f[2 * w] = bf16_bits_to_f32(raw[w] & 0xffffu);
            f[2 * w + 1] = __builtin_bit_cast(float, raw[w] & 0xffff0000u);
        }
    }
    __device__ static void store(uint16_t *dst, const float *f, int n) {
        for (int e = 0; e < n; e += 2) {
            const uint32_t p = pack_bf16x2(f[e], f[e + 1]);
            *(uint32_t *)(dst + e) = p;
        }
    }
};
template <> struct Elem<float> {
    static constexpr int kPerLane = 4;
    __device__ static void widen(const u32x4_t &raw, float *f) {
        // element to a scalar first: a bit cast applied directly to a vector
        // element is folded to element 0 by this compiler
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t bits = raw[w];
            f[w] = __builtin_bit_cast(float, bits);
        }
    }
    __device__ static void store(float *dst, const float *f, int n) {
        for (int e = 0; e < n; ++e) dst[e] = f[e];
    }
};

// Merge state (ms2, l2, o2) into (ms, l, o); ms values are in log2 units.
template <int EPL>
__device__ __forceinline__ void merge_state(float &ms, float &l, float *o, float ms2, float l2,
                                            const float *o2) {
    const float m = fmaxf(ms, ms2);
    const float ref = m == neg_inf() ? 0.f : m;
    const float w1 = exp2_hw(ms - ref), w2 = exp2_hw(ms2 - ref);
    l = w1 * l + w2 * l2;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = w1 * o[e] + w2 * o2[e];
    ms = m;
}

// GEN (fp32 only): rows of any width d <= D.  Lane cl of a row still holds
// columns 4 cl .. 4 cl + 3; those at or past d read as 0, so they add nothing
// to the dot products and their o stays 0.  Rows of a width that is not a
// multiple of 4 are not 16-byte aligned and are read element by element.
template <typename T, int D, bool GEN>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
    float *__restrict__ ws, const int32_t *__restrict__ key_lens, int H, int Nk, int S, float c,
    int d) {
    constexpr int EPL = Elem<T>::kPerLane;   // elements per lane (16 bytes)
    constexpr int LPR = D / EPL;             // lanes per key row
    constexpr int RPW = 64 / LPR;            // key rows per wave-wide load
    constexpr int ROWS_IT = RPW * kUnroll;   // rows per wave per iteration
    static_assert(64 % LPR == 0, "row must fit a wave");
    static_assert(!GEN || sizeof(T) == 4, "rows of any width: fp32 only");
    const int dd = GEN ? d : D;              // row length (elements)

    __shared__ float sh_o[kWaves][D];
    __shared__ float sh_ms[kWaves], sh_l[kWaves];

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane / LPR, cl = lane % LPR;
    const size_t bh = (size_t)b * H + h;
    const int kl = visible_len(key_lens, b, Nk);
    const int chunk = (kl + S - 1) / S;
    const int k_begin = min(split * chunk, kl), k_end = min(k_begin + chunk, kl);
    const T *kp = K + bh * Nk * dd + cl * EPL;
    const T *vp = V + bh * Nk * dd + cl * EPL;
    // this lane's 16 bytes of the row at p
    [[maybe_unused]] const int ncol = dd - cl * EPL;   // columns of the row this lane holds (GEN)
    auto load = [&](const T *p) -> u32x4_t {
        if constexpr (!GEN) {
            return __builtin_nontemporal_load((const u32x4_t *)p);
        } else {
            if (ncol >= EPL && (dd & 3) == 0) return __builtin_nontemporal_load((const u32x4_t *)p);
            u32x4_t r = {0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                if (e < ncol) r[e] = __builtin_nontemporal_load((const uint32_t *)p + e);
            return r;
        }
    };

    float q[EPL];
    if constexpr (GEN)
        Elem<T>::widen(load(Q + bh * dd + cl * EPL), q);
    else
        Elem<T>::widen(*(const u32x4_t *)(Q + bh * D + cl * EPL), q);

    // the running denominator is l + lc: each iteration's sum of weights is
    // added with an error-free two-sum whose rounding error accumulates in lc
    // (a chunk can hold millions of keys)
    float ms = neg_inf(), l = 0.f, lc = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    for (int base = k_begin + wave * ROWS_IT; base < k_end; base += kWaves * ROWS_IT) {
        u32x4_t kr[kUnroll], vr[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int row = base + u * RPW + rg;
            const bool in = row < k_end;
            kr[u] = in ? load(kp + (size_t)row * dd) : u32x4_t{0, 0, 0, 0};
            vr[u] = in ? load(vp + (size_t)row * dd) : u32x4_t{0, 0, 0, 0};
        }
        float s[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float kf[EPL];
            Elem<T>::widen(kr[u], kf);
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dot = fmaf(q[e], kf[e], dot);
#pragma unroll
            for (int m = 1; m < LPR; m <<= 1) dot += shfl_xor_f32(dot, m);
            s[u] = (base + u * RPW + rg) < k_end ? dot : neg_inf();
        }
        float mx = s[0];
#pragma unroll
        for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, s[u]);
        const float ms_new = fmaxf(ms, mx * c);
        const float ref = ms_new == neg_inf() ? 0.f : ms_new;
        const float alpha = exp2_hw(ms - ref);
        ms = ms_new;
        l *= alpha;
        lc *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= alpha;
        float lt = 0.f;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float p = exp2_hw(fmaf(s[u], c, -ref));
            float vf[EPL];
            Elem<T>::widen(vr[u], vf);
            lt += p;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, vf[e], o[e]);
        }
        const float ls = l + lt, bv = ls - l;
        lc += (l - (ls - bv)) + (lt - bv);
        l = ls;
    }
    l += lc;

    // merge the RPW row groups of this wave (lanes with equal cl)
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) {
        float o2[EPL];
        const float ms2 = shfl_xor_f32(ms, m), l2 = shfl_xor_f32(l, m);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o2[e] = shfl_xor_f32(o[e], m);
        merge_state<EPL>(ms, l, o, ms2, l2, o2);
    }
    if (rg == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sh_o[wave][cl * EPL + e] = o[e];
        if (cl == 0) {
            sh_ms[wave] = ms;
            sh_l[wave] = l;
        }
    }
    __syncthreads();
    // merge the waves; one thread per output column
    const size_t rec = bh * S + split;
    const size_t nrec = (size_t)gridDim.z * H * S;
    for (int col = tid; col < dd; col += kThreads) {
        float m = sh_ms[0], lw = sh_l[0], ow = sh_o[0][col];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) merge_state<1>(m, lw, &ow, sh_ms[w], sh_l[w], &sh_o[w][col]);
        ws[rec * dd + col] = ow;
        if (col == 0) {
            ws[nrec * dd + rec] = m;
            ws[nrec * dd + nrec + rec] = lw;
        }
    }
}

// one thread per column; with GEN the threads of columns at or past d write
// nothing
template <typename T, int D, bool GEN>
__global__ __launch_bounds__(D) void decode_combine_kernel(
    const float *__restrict__ ws, T *__restrict__ O, float *__restrict__ LSE, int BH, int S, int d) {
    const int bh = blockIdx.x, col = threadIdx.x;
    const int dd = GEN ? d : D;
    const size_t nrec = (size_t)BH * S;
    const float *wo = ws + (size_t)bh * S * dd;
    const float *wm = ws + nrec * dd + (size_t)bh * S;
    const float *wl = ws + nrec * dd + nrec + (size_t)bh * S;
    float m = neg_inf();
    for (int s = 0; s < S; ++s) m = fmaxf(m, wm[s]);
    const float ref = m == neg_inf() ? 0.f : m;
    float l = 0.f, o = 0.f;
    for (int s = 0; s < S; ++s) {   // fixed order: deterministic
        const float w = exp2_hw(wm[s] - ref);
        l = fmaf(w, wl[s], l);
        if (!GEN || col < dd) o = fmaf(w, wo[(size_t)s * dd + col], o);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float mine = o * inv;
    if constexpr (GEN) {
        if (col < dd) O[(size_t)bh * dd + col] = mine;
    } else {
        // pairs of columns for bf16 stores
        const float nbr = __shfl_xor(mine, 1, 64);
        if ((col & 1) == 0) {
            float pair[2] = {mine, nbr};
            Elem<T>::store(O + (size_t)bh * D + col, pair, 2);
        }
    }
    if (col == 0) LSE[bh] = l > 0.f ? (m + log2_hw(l)) * kLn2 : neg_inf();
}

template <typename T, int D, bool GEN = false>
hipError_t launch_t(const DecodeArgs &a, hipStream_t stream) {
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((decode_split_kernel<T, D, GEN>), dim3(a.num_splits, a.H, a.B), dim3(kThreads),
                       0, stream, (const T *)a.Q, (const T *)a.K, (const T *)a.V, a.workspace,
                       a.key_lens, a.H, a.Nk, a.num_splits, c, a.d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D, GEN>), dim3(a.B * a.H), dim3(D), 0, stream,
                       (const float *)a.workspace, (T *)a.O, a.LSE, a.B * a.H, a.num_splits, a.d);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, bool is_bf16, hipStream_t stream) {
    if (is_bf16) return a.d == 64 ? launch_t<uint16_t, 64>(a, stream) : launch_t<uint16_t, 128>(a, stream);
    if (a.d == 64) return launch_t<float, 64>(a, stream);
    if (a.d == 128) return launch_t<float, 128>(a, stream);
    // fp32 rows of other widths: the smallest lane layout that holds them
    if (a.d <= 16) return launch_t<float, 16, true>(a, stream);
    if (a.d <= 64) return launch_t<float, 64, true>(a, stream);
    if (a.d <= 128) return launch_t<float, 128, true>(a, stream);
    return launch_t<float, 256, true>(a, stream);
}

}  // namespace fa
