// fa_fwd_f32.hip -- fp32 prefill attention forward (any 1 <= d <= 256).
//
// The same tile recurrence as the bf16 path ('Online Softmax -- the
// mathematical heart of FlashAttention', sections 4-5), with every product and
// sum in fp32 on the vector ALUs: no reduced-precision matrix instruction
// touches the data.  One workgroup holds 64 query rows; four lanes share a row
// and split its d dimension in 4-float pieces, so a score is four partial dot
// products combined by two lane exchanges inside the quad.  K/V tiles of 32
// keys are staged in LDS, zero-padded to the compiled width DMAX (zeros add
// nothing to a dot product and the padded output columns are never stored).
// Fully masked rows give O = 0 and LSE = -inf as in the bf16 path.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = kThreads / 4;   // query rows per workgroup
constexpr int kBc = 32;               // keys per tile

template <int DMAX>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, const int32_t *__restrict__ key_lens,
    int H, int N, int Nk, int d, int causal, int n_qtiles, float c) {
    constexpr int NCH = DMAX / 16;    // 4-float pieces per lane
    __shared__ __attribute__((aligned(16))) float Ks[kBc * DMAX];
    __shared__ __attribute__((aligned(16))) float Vs[kBc * DMAX];

    const int tid = threadIdx.x, part = tid & 3;
    const int qtile = blockIdx.x % n_qtiles, bh = blockIdx.x / n_qtiles, b = bh / H;
    const int qrow = qtile * kRows + (tid >> 2);
    const int off = Nk - N;
    const int kv_lim = visible_len(key_lens, b, Nk);
    int kv_end = kv_lim;
    if (causal) kv_end = min(kv_end, min(qtile * kRows + kRows, N) - 1 + off + 1);
    const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;
    const size_t q_base = (size_t)bh * N * d, kv_base = (size_t)bh * Nk * d;

    float q[NCH][4], o[NCH][4];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 16 * k + 4 * part + e;
            q[k][e] = (qrow < N && col < d) ? Q[q_base + (size_t)qrow * d + col] : 0.f;
            o[k][e] = 0.f;
        }
    float ms = neg_inf(), l = 0.f;

    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * kBc;
        __syncthreads();   // previous tile fully consumed
        for (int e = tid; e < kBc * DMAX; e += kThreads) {
            const int row = e / DMAX, col = e % DMAX, j = j0 + row;
            const bool in = j < kv_end && col < d;
            Ks[e] = in ? K[kv_base + (size_t)j * d + col] : 0.f;
            Vs[e] = in ? V[kv_base + (size_t)j * d + col] : 0.f;
        }
        __syncthreads();

        float s[kBc];
#pragma unroll
        for (int jj = 0; jj < kBc; ++jj) {
            float part_dot = 0.f;
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const f32x4_t kv = *(const f32x4_t *)&Ks[jj * DMAX + 16 * k + 4 * part];
#pragma unroll
                for (int e = 0; e < 4; ++e) part_dot = fmaf(q[k][e], kv[e], part_dot);
            }
            part_dot += shfl_xor_f32(part_dot, 1);
            part_dot += shfl_xor_f32(part_dot, 2);
            const int key = j0 + jj;
            const bool ok = key < kv_lim && (!causal || key <= qrow + off);
            s[jj] = ok ? part_dot : neg_inf();
        }
        float mx = s[0];
#pragma unroll
        for (int jj = 1; jj < kBc; ++jj) mx = fmaxf(mx, s[jj]);
        const float ms_new = fmaxf(ms, mx * c);
        const float ms_ref = ms_new == neg_inf() ? 0.f : ms_new;   // -inf guard
        const float alpha = exp2_hw(ms - ms_ref);
        ms = ms_new;
        l *= alpha;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[k][e] *= alpha;
#pragma unroll
        for (int jj = 0; jj < kBc; ++jj) {
            const float p = exp2_hw(fmaf(s[jj], c, -ms_ref));
            l += p;
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const f32x4_t vv = *(const f32x4_t *)&Vs[jj * DMAX + 16 * k + 4 * part];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[k][e] = fmaf(p, vv[e], o[k][e]);
            }
        }
    }

    if (qrow < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = 16 * k + 4 * part + e;
                if (col < d) O[q_base + (size_t)qrow * d + col] = o[k][e] * inv;
            }
        if (part == 0)
            LSE[(size_t)bh * N + qrow] = l > 0.f ? (ms + log2_hw(l)) * kLn2 : neg_inf();
    }
}

template <int DMAX>
hipError_t launch_one(const FwdArgs &a, hipStream_t stream) {
    const int n_qtiles = (a.N + kRows - 1) / kRows;
    const long long nblocks = (long long)a.B * a.H * n_qtiles;
    hipLaunchKernelGGL(fwd_f32_kernel<DMAX>, dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                       (const float *)a.Q, (const float *)a.K, (const float *)a.V, (float *)a.O,
                       a.LSE, a.key_lens, a.H, a.N, a.Nk, a.d, a.causal, n_qtiles,
                       a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream) {
    if (a.d <= 16) return launch_one<16>(a, stream);
    if (a.d <= 64) return launch_one<64>(a, stream);
    if (a.d <= 128) return launch_one<128>(a, stream);
    return launch_one<256>(a, stream);
}

}  // namespace fa
