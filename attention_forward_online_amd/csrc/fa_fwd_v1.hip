// fa_fwd_v1.hip -- the FlashAttention V1 loop order, kept as an ablation.
//
// 'Online Softmax & FlashAttention' (interview lesson), Step 2: the key/value
// blocks form the outer loop and the query blocks the inner one; for every
// (key block, query block) pair the normalised output O and the row
// statistics (m, l) are read from HBM, merged with the block's contribution
// and written back:
//     m_new = max(m_old, rowmax(S)),  l_new = exp(m_old - m_new) l_old + rowsum(exp(S - m_new)),
//     O_new = (l_old exp(m_old - m_new) O_old + exp(S - m_new) V) / l_new
// (the page's exp(m_ij - m_new) P_ij with P_ij = exp(S - m_ij) is folded into
// one exponential against m_new).  Parallelism is one workgroup per (batch,
// head), as in V1.  The tile arithmetic is the V2 kernel's (fa_fwd_bf16.hip):
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16, the perm32 key order, V^T from the
// LDS transpose read; only the loop order, the state round trips through HBM
// (fp32 O, m, l in the caller's workspace) and the per-block division differ,
// so timing the two isolates what the page says V2 saves.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 128;     // query rows per inner block (32 per wave)
constexpr int kBc = 64;      // keys per outer block
constexpr int kPad = 8;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_v1_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ O, float *__restrict__ LSE, const int32_t *__restrict__ key_lens,
    float *__restrict__ Ost, float *__restrict__ Mst, float *__restrict__ Lst, int H, int N, int Nk,
    float c) {
    constexpr int KS = D + kPad;
    constexpr int KK = D / 16;
    constexpr int CB = D / 32;
    constexpr int KL = kBc * D / 8 / kThreads;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kBc * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[kBc * KS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, g = lane >> 5;
    const int krow = perm32(li);
    const int vrow = (li & 15) >> 2;
    const int vcol = perm32(4 * ((li & 3) + 4 * (li >> 4)));
    const __attribute__((address_space(3))) uint16_t *vs_lds =
        (const __attribute__((address_space(3))) uint16_t *)&Vs[0];

    const int bh = blockIdx.x, b = bh / H;
    const int off = Nk - N;
    const int kv_lim = visible_len(key_lens, b, Nk);
    int kv_end = kv_lim;
    if (CAUSAL) kv_end = min(kv_end, max(N + off, 0));   // keys some query sees
    const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;
    const int nq = (N + kBr - 1) / kBr;
    const size_t q_base = (size_t)bh * N * D, kv_base = (size_t)bh * Nk * D;
    const rsrc_t qsrc = make_rsrc(Q + q_base, (uint32_t)N * D * 2);
    const rsrc_t ksrc = make_rsrc(K + kv_base, (uint32_t)max(kv_end, 0) * D * 2);
    const rsrc_t vsrc = make_rsrc(V + kv_base, (uint32_t)max(kv_end, 0) * D * 2);
    float *ost = Ost + q_base;
    float *mst = Mst + (size_t)bh * N;
    float *lst = Lst + (size_t)bh * N;

    for (int t = 0; t < ntiles; ++t) {          // outer: one key/value block in LDS
        const int j0 = t * kBc;
        {
            u32x4_t kr[KL], vr[KL];
#pragma unroll
            for (int p = 0; p < KL; ++p) {
                const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
                const uint32_t ob = (uint32_t)((j0 + row) * D + 8 * col8) * 2;
                kr[p] = buffer_load16(ksrc, ob);
                vr[p] = buffer_load16(vsrc, ob);
            }
            __syncthreads();                    // everyone is done with the previous block
#pragma unroll
            for (int p = 0; p < KL; ++p) {
                const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
                *(u32x4_t *)&Ks[row * KS + 8 * col8] = kr[p];
                *(u32x4_t *)&Vs[row * KS + 8 * col8] = vr[p];
            }
            __syncthreads();
        }
        const int ib0 = CAUSAL ? max(0, j0 - off) / kBr : 0;
        for (int ib = ib0; ib < nq; ++ib) {     // inner: sweep the query blocks
            const int wq_first = ib * kBr + wave * 32;
            const int wq_last = min(wq_first + 32, N) - 1;
            if (wq_first > wq_last || (CAUSAL && j0 > wq_last + off)) continue;   // wave-uniform
            const int qrow = wq_first + li;
            u32x4_t qf[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                qf[kk] = buffer_load16(qsrc, (uint32_t)(qrow * D + 16 * kk + 8 * g) * 2);
            // state of these rows from HBM (none before the first block: every
            // row that sees a key sees key 0, so it is first visited at t = 0)
            float m_old = neg_inf(), l_old = 0.f;
            f32x16_t acc[CB];
            if (t > 0 && qrow < N) {
                m_old = mst[qrow];
                l_old = lst[qrow];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const f32x4_t a = *(const f32x4_t *)(ost + (size_t)qrow * D + 32 * cb + 16 * h + 8 * g);
                        const f32x4_t bq = *(const f32x4_t *)(ost + (size_t)qrow * D + 32 * cb + 16 * h + 8 * g + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            acc[cb][8 * h + e] = a[e];
                            acc[cb][8 * h + 4 + e] = bq[e];
                        }
                    }
            } else {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
            }
            wait_vmem_all();
            f32x16_t sc[2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const uint16_t *kp = &Ks[(32 * jb + krow) * KS + 8 * g];
                sc[jb] = mfma32(*(const u32x4_t *)kp, qf[0], f32x16_t{});
#pragma unroll
                for (int kk = 1; kk < KK; ++kk)
                    sc[jb] = mfma32(*(const u32x4_t *)(kp + 16 * kk), qf[kk], sc[jb]);
            }
            const bool need_mask = (j0 + kBc > kv_lim) || (CAUSAL && j0 + kBc - 1 > wq_first + off);
            if (need_mask) {
                const int vis_end = CAUSAL ? min(kv_lim, qrow + off + 1) : kv_lim;
                const int lim = vis_end - j0 - 8 * g;
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (32 * jb + 16 * (v >> 3) + (v & 7) >= lim) sc[jb][v] = neg_inf();
            }
            float mx = neg_inf();
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[jb][v]);
            mx = max_xor32(mx) * c;                 // log2 units, whole 64-key row
            const float m_new = fmaxf(m_old, mx);
            const float ms = m_new == neg_inf() ? 0.f : m_new;
            uint32_t pk[2][8];
            float lb = 0.f;
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const float p0 = exp2_hw(fmaf(sc[jb][v], c, -ms));
                    const float p1 = exp2_hw(fmaf(sc[jb][v + 1], c, -ms));
                    lb += p0 + p1;
                    pk[jb][v >> 1] = pack_bf16x2(p0, p1);
                }
            lb += shfl_xor_f32(lb, 32);
            const float alpha = m_old == neg_inf() ? 0.f : exp2_hw(m_old - ms);
            const float l_new = alpha * l_old + lb;
            // O_old back to an unnormalised sum, add P V, divide by the new l
            const float back = alpha * l_old;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[cb][v] *= back;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const auto *p0 = vs_lds + (8 * g + vrow + 32 * jb + 16 * h) * KS + vcol + 32 * cb;
                        const u32x2_t lo = lds_read_tr16(p0);
                        const u32x2_t hi = lds_read_tr16(p0 + 4 * KS);
                        acc[cb] = mfma32(u32x4_t{lo[0], lo[1], hi[0], hi[1]},
                                         u32x4_t{pk[jb][4 * h], pk[jb][4 * h + 1], pk[jb][4 * h + 2],
                                                 pk[jb][4 * h + 3]},
                                         acc[cb]);
                    }
            const float inv = l_new > 0.f ? 1.f / l_new : 0.f;
            if (qrow < N) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        f32x4_t a, bq;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            a[e] = acc[cb][8 * h + e] * inv;
                            bq[e] = acc[cb][8 * h + 4 + e] * inv;
                        }
                        *(f32x4_t *)(ost + (size_t)qrow * D + 32 * cb + 16 * h + 8 * g) = a;
                        *(f32x4_t *)(ost + (size_t)qrow * D + 32 * cb + 16 * h + 8 * g + 4) = bq;
                    }
                if (g == 0) {
                    mst[qrow] = m_new;
                    lst[qrow] = l_new;
                }
            }
        }
    }
    // O is already normalised: convert it; rows that never saw a key get 0, -inf
    __syncthreads();
    for (int r = tid; r < N * (D / 8); r += kThreads) {
        const int row = r / (D / 8), c8 = r % (D / 8);
        const int vis = CAUSAL ? min(kv_lim, row + off + 1) : kv_lim;
        u32x4_t w = u32x4_t{0u, 0u, 0u, 0u};
        if (vis > 0) {
            const f32x4_t a = *(const f32x4_t *)(ost + (size_t)row * D + 8 * c8);
            const f32x4_t bq = *(const f32x4_t *)(ost + (size_t)row * D + 8 * c8 + 4);
            w = u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(bq[0], bq[1]),
                        pack_bf16x2(bq[2], bq[3])};
        }
        *(u32x4_t *)(O + q_base + (size_t)row * D + 8 * c8) = w;
        if (c8 == 0) {
            const float l = vis > 0 ? lst[row] : 0.f;
            LSE[(size_t)bh * N + row] = l > 0.f ? (mst[row] + log2_hw(l)) * kLn2 : neg_inf();
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_v1_t(const FwdArgs &a, void *workspace, hipStream_t stream) {
    const long long BH = (long long)a.B * a.H;
    float *Ost = static_cast<float *>(workspace);
    float *Mst = Ost + BH * a.N * D;
    float *Lst = Mst + BH * a.N;
    hipLaunchKernelGGL((fwd_v1_kernel<D, CAUSAL>), dim3((unsigned)BH), dim3(kThreads), 0, stream,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (uint16_t *)a.O, a.LSE, a.key_lens, Ost, Mst, Lst, a.H, a.N, a.Nk,
                       a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

size_t forward_v1_workspace_bytes(long long B, long long H, long long N, long long d) {
    return (size_t)(B * H * N * (d + 2)) * sizeof(float);
}

hipError_t launch_fwd_v1(const FwdArgs &a, void *workspace, hipStream_t stream) {
    if (a.d == 64)
        return a.causal ? launch_v1_t<64, true>(a, workspace, stream) : launch_v1_t<64, false>(a, workspace, stream);
    return a.causal ? launch_v1_t<128, true>(a, workspace, stream) : launch_v1_t<128, false>(a, workspace, stream);
}

}  // namespace fa
