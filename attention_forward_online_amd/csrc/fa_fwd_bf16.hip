// fa_fwd_bf16.hip -- bf16 prefill attention forward on gfx950 matrix cores.
//
// Structure ('Online Softmax & FlashAttention' (interview lesson), Step 3):
// one workgroup owns one block of Br = 128 query rows for the whole loop
// (independent of every other block) and streams the K/V tiles of its head
// through LDS.  For each tile it applies the tile form of the online-softmax
// recurrence ('Online Softmax -- the mathematical heart of FlashAttention',
// sections 4 and 5):
//     m_new = max(m, rowmax(S));  alpha = exp(m - m_new)
//     P = exp(S - m_new);  l = alpha * l + rowsum(P);  o = alpha * o + P V
// and divides once at the end (the deferred normalisation the research-hub
// 'Online Softmax' page attributes to FA-2), writing O = o / l and
// LSE = m + ln l.  Causal tiles wholly above the diagonal are never loaded,
// tiles on it are masked element-wise ('Online Softmax & FlashAttention',
// Step 4).  A row that sees no key keeps m = -inf: alpha and P are then
// computed against a reference of 0 (the guard of that page's Step 1), l stays
// 0 and the epilogue writes O = 0, LSE = -inf.
//
// gfx950 mapping (4 waves, 32 query rows per wave):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the Q fragment is the B
//     operand and stays in VGPRs for the whole loop; K rows come from LDS.
//     In the 32x32 accumulator each lane holds one query column, so a row
//     max/sum is an in-lane reduction plus one exchange with lane ^ 32.
//   * The rows of each 32-key block are read in the order perm32 (bits 2 and
//     3 of the row index swapped).  Then accumulator registers 8h..8h+7 of
//     lane half g are keys 16h + 8g + 0..7: converted to bf16 they are the B
//     operand of O^T = V^T P^T without any data movement, and the matching
//     A operand is one 16-byte read of V^T from LDS.
//   * V is transposed on its way into LDS (4x8 blocks, v_perm), K is copied.
//   * Scores stay fp32; exp runs as 2^(s*scale*log2 e - m'), one FMA plus
//     v_exp_f32 per score; P is rounded to bf16 (RNE) only as the MFMA operand
//     while the row sum uses the fp32 values.
//   * Two LDS stages: the next tile's global loads are in flight while the
//     current tile is computed; one barrier per tile.
//   * Workgroup order: all Q blocks of a head run on one XCD (the dispatcher
//     deals workgroups to the 8 XCDs round-robin), so K/V re-reads of that
//     head hit the same L2; causal launches start with the longest blocks.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBc = 64;                     // keys per K/V tile
constexpr int kKPad = 8;                    // bf16 pad per K row in LDS
constexpr int kVPad = 8;                    // bf16 pad per V^T row in LDS

// Operand row r of a 32-row MFMA block reads key (or V column) perm32(r).
__device__ __forceinline__ int perm32(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE,
    const int32_t *__restrict__ key_lens, int H, int N, int Nk, int n_qtiles,
    int xcd_groups, float c) {
    constexpr int KS = D + kKPad;               // K row stride in LDS (elements)
    constexpr int VS = kBc + kVPad;             // V^T row stride in LDS
    constexpr int KK = D / 16;                  // k-steps of S^T = K Q^T
    constexpr int CB = D / 32;                  // 32-column blocks of O^T
    constexpr int KCH = kBc * D / 8;            // 16-byte chunks per K tile
    constexpr int KL = KCH / kThreads;          // ... per thread
    constexpr int VBLK = (kBc / 4) * (D / 8);   // 4x8 blocks per V tile
    static_assert(KCH % kThreads == 0 && VBLK <= kThreads, "tile/thread mismatch");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBc * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, g = lane >> 5;

    // workgroup -> (head, query block)
    const int BH = gridDim.x / n_qtiles;
    const int bid = blockIdx.x;
    int qt_rank, bh;
    if (xcd_groups) {               // B*H divisible by 8: heads grouped per XCD
        const int hpx = BH >> 3, slot = bid >> 3;
        qt_rank = slot / hpx;
        bh = (bid & 7) * hpx + slot % hpx;
    } else {
        qt_rank = bid / BH;
        bh = bid % BH;
    }
    const int qtile = CAUSAL ? (n_qtiles - 1 - qt_rank) : qt_rank;
    const int b = bh / H;
    const int q0 = qtile * kBr;
    const int off = Nk - N;                     // causal: key j visible to query i iff j <= i + off
    const int kv_lim = visible_len(key_lens, b, Nk);
    int kv_end = kv_lim;
    if (CAUSAL) kv_end = min(kv_end, min(q0 + kBr, N) - 1 + off + 1);
    const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;

    const size_t q_base = (size_t)bh * N * D;
    const size_t kv_base = (size_t)bh * Nk * D;
    const int wq_first = q0 + wave * kRowsPerWave;
    const int wq_last = min(wq_first + kRowsPerWave, N) - 1;   // < wq_first: wave has no rows
    const int qrow = wq_first + li;

    u32x4_t qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = qrow < N ? *(const u32x4_t *)(Q + q_base + (size_t)qrow * D + 16 * kk + 8 * g)
                          : u32x4_t{0, 0, 0, 0};

    f32x16_t acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
    float ms = neg_inf();   // running max of scale*log2(e)*score
    float l = 0.f;          // this lane's half of the running denominator

    u32x4_t kreg[KL];
    u32x4_t vreg[4];

    auto gload = [&](int t) {
        const int j0 = t * kBc;
#pragma unroll
        for (int p = 0; p < KL; ++p) {
            const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
            const int j = j0 + row;
            kreg[p] = j < kv_end ? *(const u32x4_t *)(K + kv_base + (size_t)j * D + 8 * col8)
                                 : u32x4_t{0, 0, 0, 0};
        }
        if (tid < VBLK) {
            const int rq = tid / (D / 8), cq = tid % (D / 8);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = j0 + 4 * rq + k;
                vreg[k] = j < kv_end ? *(const u32x4_t *)(V + kv_base + (size_t)j * D + 8 * cq)
                                     : u32x4_t{0, 0, 0, 0};
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int p = 0; p < KL; ++p) {
            const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
            *(u32x4_t *)&Ks[buf][row * KS + 8 * col8] = kreg[p];
        }
        if (tid < VBLK) {
            const int rq = tid / (D / 8), cq = tid % (D / 8);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // columns 8cq+2w (low halves) and 8cq+2w+1 (high halves) of rows 4rq..4rq+3
                const uint32_t lo0 = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
                const uint32_t hi0 = (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16);
                const uint32_t lo1 = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
                const uint32_t hi1 = (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u);
                *(u32x2_t *)&Vt[buf][(8 * cq + 2 * w) * VS + 4 * rq] = u32x2_t{lo0, hi0};
                *(u32x2_t *)&Vt[buf][(8 * cq + 2 * w + 1) * VS + 4 * rq] = u32x2_t{lo1, hi1};
            }
        }
    };

    if (ntiles > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    const int krow = perm32(li);
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int j0 = t * kBc;
        if (t + 1 < ntiles) gload(t + 1);

        const bool active = wq_first <= wq_last && (!CAUSAL || j0 <= wq_last + off);
        if (active) {
            // S^T for keys j0 .. j0+63 (two 32-key blocks) x this wave's 32 queries
            f32x16_t s[2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
                for (int v = 0; v < 16; ++v) s[jb][v] = 0.f;
                const uint16_t *kp = &Ks[buf][(32 * jb + krow) * KS + 8 * g];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    s[jb] = mfma32(*(const u32x4_t *)(kp + 16 * kk), qf[kk], s[jb]);
            }
            // mask: key length, ragged end, causal diagonal
            const bool need_mask =
                (j0 + kBc > kv_lim) || (CAUSAL && j0 + kBc - 1 > wq_first + off);
            if (need_mask) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = j0 + 32 * jb + 16 * (v >> 3) + 8 * g + (v & 7);
                        const bool ok = key < kv_lim && (!CAUSAL || key <= qrow + off);
                        if (!ok) s[jb][v] = neg_inf();
                    }
            }
            // tile row max: 32 keys in-lane, the other 32 in lane ^ 32
            float mx = s[0][0];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[jb][v]);
            mx = fmaxf(mx, shfl_xor_f32(mx, 32));
            const float ms_new = fmaxf(ms, mx * c);
            const float ms_ref = ms_new == neg_inf() ? 0.f : ms_new;   // -inf guard
            const float alpha = exp2_hw(ms - ms_ref);
            ms = ms_new;

            uint32_t pk[2][8];
            float rs = 0.f;
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const float p0 = exp2_hw(fmaf(s[jb][v], c, -ms_ref));
                    const float p1 = exp2_hw(fmaf(s[jb][v + 1], c, -ms_ref));
                    rs += p0 + p1;
                    pk[jb][v >> 1] = pack_bf16x2(p0, p1);
                }
            l = l * alpha + rs;
            if (!__all(alpha == 1.f)) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[cb][v] *= alpha;
            }
            // O^T += V^T P^T
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const uint16_t *vp = &Vt[buf][(32 * cb + krow) * VS + 8 * g];
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u32x4_t bop = {pk[jb][4 * h], pk[jb][4 * h + 1], pk[jb][4 * h + 2],
                                             pk[jb][4 * h + 3]};
                        acc[cb] = mfma32(*(const u32x4_t *)(vp + 32 * jb + 16 * h), bop, acc[cb]);
                    }
            }
        }
        if (t + 1 < ntiles) lstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: O = o / l (0 for a row without keys), LSE = m + ln l (-inf then)
    const float lt = l + shfl_xor_f32(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qrow < N) {
        uint16_t *orow = O + q_base + (size_t)qrow * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4_t w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16x2(acc[cb][8 * h + 2 * e] * inv, acc[cb][8 * h + 2 * e + 1] * inv);
                *(u32x4_t *)(orow + 32 * cb + 16 * h + 8 * g) = w;
            }
        if (g == 0)
            LSE[(size_t)bh * N + qrow] = lt > 0.f ? (ms + log2_hw(lt)) * kLn2 : neg_inf();
    }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs &a, hipStream_t stream) {
    const int n_qtiles = (a.N + kBr - 1) / kBr;
    const long long BH = (long long)a.B * a.H;
    const long long nblocks = BH * n_qtiles;
    const int xcd_groups = (BH % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)nblocks), dim3(kThreads), 0,
                       stream, (const uint16_t *)a.Q, (const uint16_t *)a.K,
                       (const uint16_t *)a.V, (uint16_t *)a.O, a.LSE, a.key_lens, a.H, a.N,
                       a.Nk, n_qtiles, xcd_groups, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream) {
    if (a.d == 64) return a.causal ? launch_one<64, true>(a, stream) : launch_one<64, false>(a, stream);
    return a.causal ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
}

}  // namespace fa
