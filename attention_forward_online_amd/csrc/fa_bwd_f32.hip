// fa_bwd_f32.hip -- fp32 attention backward (1 <= d <= 256) on the vector ALUs.
//
// The gradients of fa_bwd_bf16.hip with every product and sum in fp32 and no
// matrix instruction (the fp32 forward's layout, fa_fwd_f32.hip): LPR lanes
// share a row and split its d dimension in 4-float pieces, so a dot product is
// LPR partial sums combined by lane exchanges (LPR = 4 up to d = 128, 16 beyond,
// which keeps each lane's pieces of a row at 16 floats).  P is recomputed from the
// saved LSE ('Online softmax in attention -- why and how', "Where this is
// heading"):
//     P_ij = exp(s_ij - LSE_i),  dS_ij = P_ij (dO_i . v_j - D_i),
//     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
// bwd_dq_f32_kernel: 256 / LPR query rows per workgroup stream K/V tiles of 32 keys.
// bwd_dkdv_f32_kernel: 256 / LPR keys per workgroup stream Q/dO tiles of 32 queries.
// D_i and LSE_i * log2 e come from the workspace that the preparation kernel
// fills (per head, padded to 64 rows with zeros), as in the bf16 backward.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kT = 32;                // keys / queries per streamed tile
constexpr int kPadRows = 64;          // per-head padding of the workspace arrays

__global__ __launch_bounds__(kThreads) void bwd_prep_f32_kernel(const float *__restrict__ O,
                                                                const float *__restrict__ dO,
                                                                const float *__restrict__ LSE,
                                                                float *__restrict__ L2,
                                                                float *__restrict__ Dd,
                                                                long long BH, int N, int Npad, int d) {
    const long long prow = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (prow >= BH * Npad) return;
    const long long bh = prow / Npad;
    const int i = (int)(prow % Npad);
    if (i >= N) {
        Dd[prow] = 0.f;
        L2[prow] = 0.f;
        return;
    }
    const long long row = bh * N + i;
    float acc = 0.f;
    for (int c = 0; c < d; ++c) acc = fmaf(O[row * d + c], dO[row * d + c], acc);
    const float lse = LSE[row];
    Dd[prow] = acc;
    L2[prow] = lse == neg_inf() ? 0.f : lse * kLog2e;
}

// Lane `part` of a row's LPR lanes holds columns 4 LPR k + 4 part + 0..3 of
// the row (piece k = 0 .. NCH - 1).

// sum over the LPR lanes of a row (LPR = 4: a quad; 16: a DPP row)
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(LPR == 4 || LPR == 16, "quad or DPP row");
    if constexpr (LPR == 16) {
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));   // row_ror:8
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));   // row_ror:4
    }
    x += quad_xor_f32<1>(x);
    x += quad_xor_f32<2>(x);
    return x;
}

// dot of this lane's pieces with a DMAX-wide LDS row, summed over the row's lanes
template <int LPR, int NCH>
__device__ __forceinline__ float row_dot(const float (&x)[NCH][4], const float *row, int part) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const f32x4_t y = *(const f32x4_t *)&row[4 * LPR * k + 4 * part];
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(x[k][e], y[e], s);
    }
    return row_sum<LPR>(s);
}

template <int LPR, int NCH>
__device__ __forceinline__ void axpy(float (&acc)[NCH][4], float a, const float *row, int part) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const f32x4_t y = *(const f32x4_t *)&row[4 * LPR * k + 4 * part];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k][e] = fmaf(a, y[e], acc[k][e]);
    }
}

template <int LPR, int NCH>
__device__ __forceinline__ void load_row(float (&x)[NCH][4], const float *src, bool ok, int d, int part) {
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 4 * LPR * k + 4 * part + e;
            x[k][e] = (ok && col < d) ? src[col] : 0.f;
        }
}

template <int LPR, int NCH>
__device__ __forceinline__ void store_row(float *dst, const float (&x)[NCH][4], float mul, int d, int part) {
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 4 * LPR * k + 4 * part + e;
            if (col < d) dst[col] = x[k][e] * mul;
        }
}

template <int DMAX, int LPR>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, float *__restrict__ dQ, const float *__restrict__ L2,
    const float *__restrict__ Dd, const int32_t *__restrict__ key_lens, int H, int N, int Nk,
    int Npad, int d, int causal, int n_qtiles, float c, float scale) {
    constexpr int kRows = kThreads / LPR;
    constexpr int NCH = DMAX / (4 * LPR);
    static_assert(NCH >= 1 && NCH * 4 * LPR == DMAX, "width/lane split");
    __shared__ __attribute__((aligned(16))) float Ks[kT * DMAX];
    __shared__ __attribute__((aligned(16))) float Vs[kT * DMAX];
    const int tid = threadIdx.x, part = tid % LPR;
    const int qtile = blockIdx.x % n_qtiles, bh = blockIdx.x / n_qtiles, b = bh / H;
    const int qrow = qtile * kRows + tid / LPR;
    const int off = Nk - N;
    const int kv_lim = visible_len(key_lens, b, Nk);
    int kv_end = kv_lim;
    if (causal) kv_end = min(kv_end, min(qtile * kRows + kRows, N) - 1 + off + 1);
    const int ntiles = kv_end > 0 ? (kv_end + kT - 1) / kT : 0;
    const size_t q_base = (size_t)bh * N * d, kv_base = (size_t)bh * Nk * d;
    const bool qok = qrow < N;

    float q[NCH][4], g[NCH][4], acc[NCH][4];
    load_row<LPR, NCH>(q, Q + q_base + (size_t)qrow * d, qok, d, part);
    load_row<LPR, NCH>(g, dO + q_base + (size_t)qrow * d, qok, d, part);
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k][e] = 0.f;
    const float l2 = qok ? L2[(size_t)bh * Npad + qrow] : 0.f;
    const float dd = qok ? Dd[(size_t)bh * Npad + qrow] : 0.f;

    // K/V tiles: a thread's loads are issued at once, and up to DMAX = 64
    // (where the registers allow it) the next tile's loads are in flight while
    // one is computed
    constexpr bool kPrefetch = DMAX <= 64;
    const rsrc_t ksrc = make_rsrc(K + kv_base, (uint32_t)max(kv_end, 0) * d * 4);
    const rsrc_t vsrc = make_rsrc(V + kv_base, (uint32_t)max(kv_end, 0) * d * 4);
    F32TileStage<kT, DMAX, kThreads> kst, vst;
    if (kPrefetch && ntiles > 0) {
        kst.load(ksrc, 0, d, tid);
        vst.load(vsrc, 0, d, tid);
    }
    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * kT;
        if (!kPrefetch) {
            kst.load(ksrc, j0, d, tid);
            vst.load(vsrc, j0, d, tid);
        }
        __syncthreads();
        kst.store(Ks, tid);
        vst.store(Vs, tid);
        __syncthreads();
        if (kPrefetch && t + 1 < ntiles) {
            kst.load(ksrc, j0 + kT, d, tid);
            vst.load(vsrc, j0 + kT, d, tid);
        }
        for (int jj = 0; jj < kT; ++jj) {
            const float s = row_dot<LPR, NCH>(q, &Ks[jj * DMAX], part);
            const float dp = row_dot<LPR, NCH>(g, &Vs[jj * DMAX], part);
            const int key = j0 + jj;
            const bool ok = qok && key < kv_lim && (!causal || key <= qrow + off);
            const float p = ok ? exp2_hw(fmaf(s, c, -l2)) : 0.f;
            axpy<LPR, NCH>(acc, p * (dp - dd), &Ks[jj * DMAX], part);
        }
    }
    if (qok) store_row<LPR, NCH>(dQ + q_base + (size_t)qrow * d, acc, scale, d, part);
}

template <int DMAX, int LPR>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, float *__restrict__ dK, float *__restrict__ dV,
    const float *__restrict__ L2, const float *__restrict__ Dd, const int32_t *__restrict__ key_lens,
    int H, int N, int Nk, int Npad, int d, int causal, int n_ktiles, float c, float scale) {
    constexpr int kRows = kThreads / LPR;
    constexpr int NCH = DMAX / (4 * LPR);
    static_assert(NCH >= 1 && NCH * 4 * LPR == DMAX, "width/lane split");
    __shared__ __attribute__((aligned(16))) float Qs[kT * DMAX];
    __shared__ __attribute__((aligned(16))) float Gs[kT * DMAX];
    __shared__ float Ls[kT], Ds[kT];
    const int tid = threadIdx.x, part = tid % LPR;
    const int ktile = blockIdx.x % n_ktiles, bh = blockIdx.x / n_ktiles, b = bh / H;
    const int k0 = ktile * kRows;
    const int key = k0 + tid / LPR;
    const int off = Nk - N;
    const int kv_lim = visible_len(key_lens, b, Nk);
    const size_t q_base = (size_t)bh * N * d, kv_base = (size_t)bh * Nk * d;
    const bool kok = key < Nk;
    // queries that see any key of this workgroup: i >= k0 - off (causal)
    const int i_first = causal ? max(0, k0 - off) : 0;
    const int ntiles = (k0 < kv_lim && i_first < N) ? (N - i_first + kT - 1) / kT : 0;

    float kr[NCH][4], vr[NCH][4], dk[NCH][4], dv[NCH][4];
    load_row<LPR, NCH>(kr, K + kv_base + (size_t)key * d, kok, d, part);
    load_row<LPR, NCH>(vr, V + kv_base + (size_t)key * d, kok, d, part);
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dk[k][e] = 0.f;
            dv[k][e] = 0.f;
        }

    // Q/dO tiles (and their LSE2, D): loads issued at once; up to DMAX = 64
    // the next tile's loads are in flight while one is computed
    constexpr bool kPrefetch = DMAX <= 64;
    const rsrc_t qsrc = make_rsrc(Q + q_base, (uint32_t)N * d * 4);
    const rsrc_t gsrc = make_rsrc(dO + q_base, (uint32_t)N * d * 4);
    const rsrc_t lsrc = make_rsrc(L2 + (size_t)bh * Npad, (uint32_t)N * 4);
    const rsrc_t dsrc = make_rsrc(Dd + (size_t)bh * Npad, (uint32_t)N * 4);
    F32TileStage<kT, DMAX, kThreads> qst, gst;
    float lv = 0.f, dv2 = 0.f;
    auto issue = [&](int i0) {
        qst.load(qsrc, i0, d, tid);
        gst.load(gsrc, i0, d, tid);
        if (tid < kT) {
            lv = buffer_load_f32(lsrc, (uint32_t)(i0 + tid) * 4);
            dv2 = buffer_load_f32(dsrc, (uint32_t)(i0 + tid) * 4);
        }
    };
    if (kPrefetch && ntiles > 0) issue(i_first);
    for (int t = 0; t < ntiles; ++t) {
        const int i0 = i_first + t * kT;
        if (!kPrefetch) issue(i0);
        __syncthreads();
        qst.store(Qs, tid);
        gst.store(Gs, tid);
        if (tid < kT) {
            Ls[tid] = lv;
            Ds[tid] = dv2;
        }
        __syncthreads();
        if (kPrefetch && t + 1 < ntiles) issue(i0 + kT);
        for (int ii = 0; ii < kT; ++ii) {
            const int i = i0 + ii;
            const float s = row_dot<LPR, NCH>(kr, &Qs[ii * DMAX], part);
            const float dp = row_dot<LPR, NCH>(vr, &Gs[ii * DMAX], part);
            const bool ok = kok && i < N && key < kv_lim && (!causal || key <= i + off);
            const float p = ok ? exp2_hw(fmaf(s, c, -Ls[ii])) : 0.f;
            axpy<LPR, NCH>(dv, p, &Gs[ii * DMAX], part);
            axpy<LPR, NCH>(dk, p * (dp - Ds[ii]), &Qs[ii * DMAX], part);
        }
    }
    if (kok) {
        store_row<LPR, NCH>(dK + kv_base + (size_t)key * d, dk, scale, d, part);
        store_row<LPR, NCH>(dV + kv_base + (size_t)key * d, dv, 1.f, d, part);
    }
}

template <int DMAX, int LPR>
hipError_t launch_t(const BwdArgs &a, hipStream_t stream) {
    constexpr int kRows = kThreads / LPR;
    const long long BH = (long long)a.B * a.H;
    const int Npad = (a.N + kPadRows - 1) / kPadRows * kPadRows;
    float *L2 = static_cast<float *>(a.workspace);
    float *Dd = L2 + BH * Npad;
    const float c = a.scale * kLog2e;
    if (a.N > 0) {
        const long long prows = BH * Npad;
        hipLaunchKernelGGL(bwd_prep_f32_kernel, dim3((unsigned)((prows + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, (const float *)a.O, (const float *)a.dO, a.LSE,
                           L2, Dd, BH, a.N, Npad, a.d);
        const int n_qt = (a.N + kRows - 1) / kRows;
        hipLaunchKernelGGL((bwd_dq_f32_kernel<DMAX, LPR>), dim3((unsigned)(BH * n_qt)), dim3(kThreads), 0,
                           stream, (const float *)a.Q, (const float *)a.K, (const float *)a.V,
                           (const float *)a.dO, (float *)a.dQ, L2, Dd, a.key_lens, a.H, a.N, a.Nk,
                           Npad, a.d, a.causal, n_qt, c, a.scale);
    }
    if (a.Nk > 0) {
        const int n_kt = (a.Nk + kRows - 1) / kRows;
        hipLaunchKernelGGL((bwd_dkdv_f32_kernel<DMAX, LPR>), dim3((unsigned)(BH * n_kt)), dim3(kThreads), 0,
                           stream, (const float *)a.Q, (const float *)a.K, (const float *)a.V,
                           (const float *)a.dO, (float *)a.dK, (float *)a.dV, L2, Dd, a.key_lens,
                           a.H, a.N, a.Nk, Npad, a.d, a.causal, n_kt, c, a.scale);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t stream) {
    if (a.d <= 16) return launch_t<16, 4>(a, stream);
    if (a.d <= 64) return launch_t<64, 4>(a, stream);
    if (a.d <= 128) return launch_t<128, 4>(a, stream);
    return launch_t<256, 16>(a, stream);
}

}  // namespace fa
