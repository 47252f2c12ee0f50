// fa_bwd_bf16.hip -- bf16 attention backward (d = 64, 128) on gfx950 matrix cores.
//
// The gradients of L = sum dO . O for the forward of fa_fwd_bf16.hip, with the
// probabilities recomputed from the saved row log-sum-exp instead of being
// read back ('Online softmax in attention -- why and how', "Where this is
// heading": backward recomputes the scores from the cached row statistics):
//     P_ij = exp(s_ij - LSE_i)          (final probabilities: no running max)
//     D_i  = dO_i . O_i
//     dS_ij = P_ij (dO_i . v_j - D_i)
//     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//     dV_j = sum_i P_ij dO_i.
// Three kernels, no atomics:
//   bwd_prep_kernel   D_i and LSE_i in log2 units (0 for a row with no key).
//   bwd_dq_kernel     one workgroup per 128 queries streams the K/V tiles (the
//                     forward's shape): S^T = K Q^T and dP^T = V dO^T with the
//                     query in the lane, then dQ^T += K^T dS^T with the K^T
//                     operand from the LDS transpose read.
//   bwd_dkdv_kernel   one workgroup per 128 keys (K and V fragments stay in
//                     VGPRs) streams the Q/dO tiles: S = Q K^T and dP = dO V^T
//                     with the key in the lane; reading the Q/dO rows in perm32
//                     order makes P and dS the B operand of dV^T += dO^T P and
//                     dK^T += Q^T dS directly, dO^T and Q^T come from transpose
//                     reads, and each lane ends with 16-byte pieces of its key's
//                     dK and dV rows.
// Masking follows the forward exactly: causal key j <= i + (Nk - N), keys at
// or past key_lens[b] invisible; invisible pairs get P = 0, hence dS = 0.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBq = 128;     // queries per dQ workgroup (32 per wave)
constexpr int kBk = 128;     // keys per dK/dV workgroup (32 per wave)
constexpr int kTile = 64;    // keys per K/V tile (dQ) and queries per Q/dO tile (dK/dV)

// LDS row stride (bf16 elements) of the Q, dO, K and V tiles.  Each tile is
// read two ways: 16-byte row reads (16 lanes per LDS pass, 16 different rows,
// conflict-free when rows step by 4 x odd banks modulo 64) and
// ds_read_b64_tr_b16 (32 lanes per pass: four consecutive rows of 16 banks
// each).  No stride serves both without conflicts; d = 64 rows step by 36
// banks (transpose reads 2-way), d = 128 rows by 76 = 12 mod 64 (transpose
// reads 2-way instead of the 4-way of a 16-byte pad).  An XOR swizzle that is
// conflict-free for both measured slower at d = 64 (more address registers).
template <int D> constexpr int kRowElems = D == 64 ? D + 8 : D + 24;
template <int D>
__device__ __forceinline__ int lds_at(int row, int col) { return row * kRowElems<D> + col; }

// Workgroup -> (head, block rank); with B*H divisible by 8 all blocks of a
// head run on one XCD (round-robin dispatch), as in the forward.
__device__ __forceinline__ void block_of(int bid, int nblk, int xcd_interleave, int &bh, int &rank) {
    const int BH = gridDim.x / nblk;
    if (xcd_interleave) {
        const int hpx = BH >> 3, slot = bid >> 3;
        rank = slot / hpx;
        bh = (slot % hpx) * 8 + (bid & 7);
    } else {
        rank = bid / BH;
        bh = bid % BH;
    }
}

// D_i = dO_i . O_i and LSE_i * log2(e) (0 when LSE_i = -inf: that row sees no
// key, so every one of its scores is masked anyway), into per-head arrays of
// Npad = N rounded up to the 64-query tile; the padding gets zeros (its
// queries are masked in every kernel).  D / 8 lanes per row.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const uint16_t *__restrict__ O,
                                                            const uint16_t *__restrict__ dO,
                                                            const float *__restrict__ LSE,
                                                            float *__restrict__ L2,
                                                            float *__restrict__ Dd, long long BH,
                                                            int N, int Npad) {
    constexpr int LPR = D / 8;
    const long long prow = ((long long)blockIdx.x * kThreads + threadIdx.x) / LPR;
    const int sub = threadIdx.x % LPR;
    if (prow >= BH * Npad) return;   // whole row groups leave together
    const long long bh = prow / Npad;
    const int i = (int)(prow % Npad);
    if (i >= N) {
        if (sub == 0) {
            Dd[prow] = 0.f;
            L2[prow] = 0.f;
        }
        return;
    }
    const long long row = bh * N + i;
    const u32x4_t o = *(const u32x4_t *)(O + row * D + 8 * sub);
    const u32x4_t g = *(const u32x4_t *)(dO + row * D + 8 * sub);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t ow = o[w], gw = g[w];
        acc = fmaf(bf16_bits_to_f32(ow & 0xffffu), bf16_bits_to_f32(gw & 0xffffu), acc);
        acc = fmaf(__builtin_bit_cast(float, ow & 0xffff0000u),
                   __builtin_bit_cast(float, gw & 0xffff0000u), acc);
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += shfl_xor_f32(acc, off);
    if (sub == 0) {
        const float lse = LSE[row];
        Dd[prow] = acc;
        L2[prow] = lse == neg_inf() ? 0.f : lse * kLog2e;
    }
}

// dQ: 4 waves x 32 queries, K/V tiles of 64 keys through two LDS stages.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO, uint16_t *__restrict__ dQ,
    const float *__restrict__ L2, const float *__restrict__ Dd,
    const int32_t *__restrict__ key_lens, int H, int N, int Nk, int Npad, int n_qtiles,
    int xcd_interleave, float c, float scale) {
    constexpr int NST = 2;
    constexpr int TILE = kTile * kRowElems<D>;
    constexpr int KK = D / 16;
    constexpr int CB = D / 32;
    constexpr int KL = kTile * D / 8 / kThreads;
    static_assert(kTile * D / 8 % kThreads == 0, "tile/thread mismatch");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[NST * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[NST * TILE];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, g = lane >> 5;
    const int krow = perm32(li);
    // K^T operand through the transpose read (the forward's V^T read): lane li
    // receives K column perm32(li) of 4 consecutive keys per read
    const int trow = (li & 15) >> 2;
    const int tcol = perm32(4 * ((li & 3) + 4 * (li >> 4)));
    const __attribute__((address_space(3))) uint16_t *ks_lds =
        (const __attribute__((address_space(3))) uint16_t *)&Ks[0];

    int bh, rank;
    block_of(blockIdx.x, n_qtiles, xcd_interleave, bh, rank);
    const int b = bh / H;
    const int off = Nk - N;
    const int kv_lim = visible_len(key_lens, b, Nk);
    const size_t q_base = (size_t)bh * N * D;
    const size_t kv_base = (size_t)bh * Nk * D;

    const int qtile = CAUSAL ? n_qtiles - 1 - rank : rank;
    const int q0 = qtile * kBq;
    int kv_end = kv_lim;
    if (CAUSAL) kv_end = min(kv_end, min(q0 + kBq, N) - 1 + off + 1);
    const int ntiles = kv_end > 0 ? (kv_end + kTile - 1) / kTile : 0;
    const int wq_first = q0 + wave * 32;
    const int wq_last = min(wq_first + 32, N) - 1;
    const int qrow = wq_first + li;

    const rsrc_t qsrc = make_rsrc(Q + q_base, (uint32_t)N * D * 2);
    const rsrc_t dosrc = make_rsrc(dO + q_base, (uint32_t)N * D * 2);
    const rsrc_t ksrc = make_rsrc(K + kv_base, (uint32_t)max(kv_end, 0) * D * 2);
    const rsrc_t vsrc = make_rsrc(V + kv_base, (uint32_t)max(kv_end, 0) * D * 2);

    u32x4_t qf[KK], dof[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qf[kk] = buffer_load16(qsrc, (uint32_t)(qrow * D + 16 * kk + 8 * g) * 2);
        dof[kk] = buffer_load16(dosrc, (uint32_t)(qrow * D + 16 * kk + 8 * g) * 2);
    }
    // a query past N takes l2 = +inf: every P of its row is 0
    float l2 = __builtin_inff(), dd = 0.f;
    if (qrow < N) {
        l2 = L2[(size_t)bh * Npad + qrow];
        dd = Dd[(size_t)bh * Npad + qrow];
    }
    wait_vmem_all();

    f32x16_t acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;

    u32x4_t kr[KL], vr[KL];
    auto gload = [&](int t) {
        const int j0 = t * kTile;
#pragma unroll
        for (int p = 0; p < KL; ++p) {
            const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
            const uint32_t off_b = (uint32_t)((j0 + row) * D + 8 * col8) * 2;
            kr[p] = buffer_load16(ksrc, off_b);
            vr[p] = buffer_load16(vsrc, off_b);
        }
    };
    auto lstore = [&](int stage) {
#pragma unroll
        for (int p = 0; p < KL; ++p) {
            const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
            *(u32x4_t *)&Ks[stage * TILE + lds_at<D>(row, 8 * col8)] = kr[p];
            *(u32x4_t *)&Vs[stage * TILE + lds_at<D>(row, 8 * col8)] = vr[p];
        }
    };
    auto active = [&](int t) {
        return wq_first <= wq_last && (!CAUSAL || t * kTile <= wq_last + off);
    };
    // X^T = R F^T for one 64-key tile: R rows (keys, perm32 order) from LDS,
    // F the per-lane query fragment
    auto rows_times = [&](const uint16_t *R, int stage, const u32x4_t (&F)[KK], f32x16_t (&s)[2]) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const uint16_t *rp = &R[stage * TILE];
            s[jb] = mfma32(*(const u32x4_t *)&rp[lds_at<D>(32 * jb + krow, 8 * g)], F[0], f32x16_t{});
#pragma unroll
            for (int kk = 1; kk < KK; ++kk)
                s[jb] = mfma32(*(const u32x4_t *)&rp[lds_at<D>(32 * jb + krow, 16 * kk + 8 * g)], F[kk], s[jb]);
        }
    };
    auto kt_operand = [&](int stage, int cb, int jb, int h) {
        const int r0 = 8 * g + trow + 32 * jb + 16 * h;
        const u32x2_t lo = lds_read_tr16(ks_lds + stage * TILE + lds_at<D>(r0, tcol + 32 * cb));
        const u32x2_t hi = lds_read_tr16(ks_lds + stage * TILE + lds_at<D>(r0 + 4, tcol + 32 * cb));
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };

    gload(0);
    lstore(0);
    gload(1);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        if (active(t)) {
            f32x16_t s[2], dp[2];
            rows_times(Ks, cur, qf, s);
            rows_times(Vs, cur, dof, dp);
            const int j0 = t * kTile;
            const bool need_mask = (j0 + kTile > kv_lim) || (CAUSAL && j0 + kTile - 1 > wq_first + off);
            if (need_mask) {
                // register v of block jb holds key j0 + 32jb + 16(v/8) + 8g + v%8
                const int vis_end = CAUSAL ? min(kv_lim, qrow + off + 1) : kv_lim;
                const int lim = vis_end - j0 - 8 * g;
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (32 * jb + 16 * (v >> 3) + (v & 7) >= lim) s[jb][v] = neg_inf();
            }
            uint32_t pk[2][8];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const float p0 = exp2_hw(fmaf(s[jb][v], c, -l2));
                    const float p1 = exp2_hw(fmaf(s[jb][v + 1], c, -l2));
                    pk[jb][v >> 1] = pack_bf16x2(p0 * (dp[jb][v] - dd), p1 * (dp[jb][v + 1] - dd));
                }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        acc[cb] = mfma32(kt_operand(cur, cb, jb, h),
                                         u32x4_t{pk[jb][4 * h], pk[jb][4 * h + 1], pk[jb][4 * h + 2],
                                                 pk[jb][4 * h + 3]},
                                         acc[cb]);
        }
        lstore(cur ^ 1);
        gload(t + 2);
        __syncthreads();
    }

    if (qrow < N) {
        uint16_t *grow = dQ + q_base + (size_t)qrow * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4_t w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16x2(acc[cb][8 * h + 2 * e] * scale, acc[cb][8 * h + 2 * e + 1] * scale);
                *(u32x4_t *)(grow + 32 * cb + 16 * h + 8 * g) = w;
            }
    }
}

// dK, dV: 4 waves x 32 keys; Q/dO tiles of 64 queries through two LDS stages.
// MODE 0 computes both; at d = 128 both accumulators do not fit next to the
// operands, so MODE 1 (dV only: S, P, dV) and MODE 2 (dK only: S, dP, dS, dK)
// run as two launches.
enum { kBoth = 0, kOnlyDV = 1, kOnlyDK = 2 };
template <int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, const float *__restrict__ L2, const float *__restrict__ Dd,
    const int32_t *__restrict__ key_lens, int H, int N, int Nk, int Npad, int n_ktiles,
    int xcd_interleave, float c, float scale) {
    constexpr int NST = 2;
    constexpr int TILE = kTile * kRowElems<D>;
    constexpr int KK = D / 16;
    constexpr int CB = D / 32;
    constexpr int KL = kTile * D / 8 / kThreads;
    constexpr bool WANT_DV = MODE != kOnlyDK, WANT_DK = MODE != kOnlyDV;
    static_assert(kTile * D / 8 % kThreads == 0, "tile/thread mismatch");

    __shared__ __attribute__((aligned(16))) uint16_t Qs[NST * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Gs[NST * TILE];   // dO
    __shared__ __attribute__((aligned(16))) float Ls[NST * kTile];
    __shared__ __attribute__((aligned(16))) float Ds[NST * kTile];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, g = lane >> 5;
    const int qperm = perm32(li);
    const int trow = (li & 15) >> 2;
    const int tcol = perm32(4 * ((li & 3) + 4 * (li >> 4)));
    const __attribute__((address_space(3))) uint16_t *qs_lds =
        (const __attribute__((address_space(3))) uint16_t *)&Qs[0];
    const __attribute__((address_space(3))) uint16_t *gs_lds =
        (const __attribute__((address_space(3))) uint16_t *)&Gs[0];

    int bh, rank;
    block_of(blockIdx.x, n_ktiles, xcd_interleave, bh, rank);
    const int b = bh / H;
    const int off = Nk - N;
    const int kv_lim = visible_len(key_lens, b, Nk);
    const size_t q_base = (size_t)bh * N * D;
    const size_t kv_base = (size_t)bh * Nk * D;

    // causal blocks that see the most queries (the first keys) go first
    const int ktile = rank;
    const int k0 = ktile * kBk;
    const int wk0 = k0 + wave * 32;
    const int key = wk0 + li;                  // this lane's key (S and dK/dV column)
    const bool key_vis = key < kv_lim;
    // queries that see any key of this workgroup: i >= k0 - off (causal)
    const int i_first = CAUSAL ? max(0, k0 - off) : 0;
    const int t_first = k0 < kv_lim ? i_first / kTile : 0;
    const int n_q = (N + kTile - 1) / kTile;
    const int ntiles = (k0 < kv_lim && i_first < N) ? n_q - t_first : 0;

    const rsrc_t ksrc = make_rsrc(K + kv_base, (uint32_t)Nk * D * 2);
    const rsrc_t vsrc = make_rsrc(V + kv_base, (uint32_t)Nk * D * 2);
    const rsrc_t qsrc = make_rsrc(Q + q_base, (uint32_t)N * D * 2);
    const rsrc_t gsrc = make_rsrc(dO + q_base, (uint32_t)N * D * 2);
    // whole tiles of the padded per-head arrays: every 16-byte load is in range
    // or (prefetch past the last tile) entirely out of it
    const rsrc_t lsrc = make_rsrc(L2 + (size_t)bh * Npad, (uint32_t)Npad * 4);
    const rsrc_t dsrc = make_rsrc(Dd + (size_t)bh * Npad, (uint32_t)Npad * 4);

    u32x4_t kf[KK], vf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        kf[kk] = buffer_load16(ksrc, (uint32_t)(key * D + 16 * kk + 8 * g) * 2);
        if constexpr (WANT_DK) vf[kk] = buffer_load16(vsrc, (uint32_t)(key * D + 16 * kk + 8 * g) * 2);
    }
    wait_vmem_all();

    f32x16_t adk[CB], adv[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            adk[cb][v] = 0.f;
            adv[cb][v] = 0.f;
        }

    u32x4_t qr[KL], gr[KL], lr = u32x4_t{0u, 0u, 0u, 0u};
    auto gload = [&](int t) {
        const int i0 = (t_first + t) * kTile;
#pragma unroll
        for (int p = 0; p < KL; ++p) {
            const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
            const uint32_t off_b = (uint32_t)((i0 + row) * D + 8 * col8) * 2;
            qr[p] = buffer_load16(qsrc, off_b);
            gr[p] = buffer_load16(gsrc, off_b);
        }
        // threads 0..15: L2 of the tile's 64 queries, 16..31: D
        if (tid < 16) lr = buffer_load16(lsrc, (uint32_t)(i0 + 4 * tid) * 4);
        else if (tid < 32) lr = buffer_load16(dsrc, (uint32_t)(i0 + 4 * (tid - 16)) * 4);
    };
    auto lstore = [&](int stage) {
#pragma unroll
        for (int p = 0; p < KL; ++p) {
            const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
            *(u32x4_t *)&Qs[stage * TILE + lds_at<D>(row, 8 * col8)] = qr[p];
            *(u32x4_t *)&Gs[stage * TILE + lds_at<D>(row, 8 * col8)] = gr[p];
        }
        if (tid < 16) *(u32x4_t *)&Ls[stage * kTile + 4 * tid] = lr;
        else if (tid < 32) *(u32x4_t *)&Ds[stage * kTile + 4 * (tid - 16)] = lr;
    };
    // a wave works on a tile if a query of it sees this wave's first key
    auto active = [&](int t) {
        const int i_last = (t_first + t) * kTile + kTile - 1;
        return wk0 < kv_lim && (!CAUSAL || i_last + off >= wk0);
    };
    // X = R F^T for the tile's 64 queries (two 32-query blocks, rows in
    // perm32 order) against this lane's key fragment F
    auto rows_times = [&](const uint16_t *R, int stage, const u32x4_t (&F)[KK], f32x16_t (&s)[2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const uint16_t *rp = &R[stage * TILE];
            s[qb] = mfma32(*(const u32x4_t *)&rp[lds_at<D>(32 * qb + qperm, 8 * g)], F[0], f32x16_t{});
#pragma unroll
            for (int kk = 1; kk < KK; ++kk)
                s[qb] = mfma32(*(const u32x4_t *)&rp[lds_at<D>(32 * qb + qperm, 16 * kk + 8 * g)], F[kk], s[qb]);
        }
    };
    // transpose read of a Q or dO tile: lane li gets column 32cb + perm32(li)
    // of queries 32qb + 16h + 8g + 0..7
    auto t_operand = [&](const __attribute__((address_space(3))) uint16_t *base, int stage, int cb,
                         int qb, int h) {
        const int r0 = 8 * g + trow + 32 * qb + 16 * h;
        const u32x2_t lo = lds_read_tr16(base + stage * TILE + lds_at<D>(r0, tcol + 32 * cb));
        const u32x2_t hi = lds_read_tr16(base + stage * TILE + lds_at<D>(r0 + 4, tcol + 32 * cb));
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };

    gload(0);
    lstore(0);
    gload(1);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        if (active(t)) {
            const int i0 = (t_first + t) * kTile;
            f32x16_t s[2], dp[2];
            rows_times(Qs, cur, kf, s);
            if constexpr (WANT_DK) rows_times(Gs, cur, vf, dp);
            // register v of block qb holds query i0 + 32qb + 16(v/8) + 8g + v%8
            const bool need_mask =
                !key_vis || (i0 + kTile > N) || (CAUSAL && i0 + off < wk0 + 31);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int i = i0 + 32 * qb + 16 * (v >> 3) + 8 * g + (v & 7);
                        if (!key_vis || i >= N || (CAUSAL && key > i + off)) s[qb][v] = neg_inf();
                    }
            }
            uint32_t pp[2][8], pd[2][8];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i8 = 32 * qb + 16 * h + 8 * g;    // 8 consecutive queries
                    const f32x4_t la = *(const f32x4_t *)&Ls[cur * kTile + i8];
                    const f32x4_t lb = *(const f32x4_t *)&Ls[cur * kTile + i8 + 4];
                    const f32x4_t da = *(const f32x4_t *)&Ds[cur * kTile + i8];
                    const f32x4_t db = *(const f32x4_t *)&Ds[cur * kTile + i8 + 4];
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const int v = 8 * h + e;
                        const float l0 = e < 4 ? la[e] : lb[e - 4], l1 = e < 4 ? la[e + 1] : lb[e - 3];
                        const float d0 = e < 4 ? da[e] : db[e - 4], d1 = e < 4 ? da[e + 1] : db[e - 3];
                        const float p0 = exp2_hw(fmaf(s[qb][v], c, -l0));
                        const float p1 = exp2_hw(fmaf(s[qb][v + 1], c, -l1));
                        if constexpr (WANT_DV) pp[qb][v >> 1] = pack_bf16x2(p0, p1);
                        if constexpr (WANT_DK)
                            pd[qb][v >> 1] = pack_bf16x2(p0 * (dp[qb][v] - d0), p1 * (dp[qb][v + 1] - d1));
                    }
                }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        if constexpr (WANT_DV)
                            adv[cb] = mfma32(t_operand(gs_lds, cur, cb, qb, h),
                                             u32x4_t{pp[qb][4 * h], pp[qb][4 * h + 1], pp[qb][4 * h + 2],
                                                     pp[qb][4 * h + 3]},
                                             adv[cb]);
                        if constexpr (WANT_DK)
                            adk[cb] = mfma32(t_operand(qs_lds, cur, cb, qb, h),
                                             u32x4_t{pd[qb][4 * h], pd[qb][4 * h + 1], pd[qb][4 * h + 2],
                                                     pd[qb][4 * h + 3]},
                                             adk[cb]);
                    }
        }
        lstore(cur ^ 1);
        gload(t + 2);
        __syncthreads();
    }

    // accumulator register 8h + e of block cb holds d = 32cb + 16h + 8g + e of this lane's key
    if (key < Nk) {
        uint16_t *krow_out = dK + kv_base + (size_t)key * D;
        uint16_t *vrow_out = dV + kv_base + (size_t)key * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4_t wk, wv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wk[e] = pack_bf16x2(adk[cb][8 * h + 2 * e] * scale, adk[cb][8 * h + 2 * e + 1] * scale);
                    wv[e] = pack_bf16x2(adv[cb][8 * h + 2 * e], adv[cb][8 * h + 2 * e + 1]);
                }
                if constexpr (WANT_DK) *(u32x4_t *)(krow_out + 32 * cb + 16 * h + 8 * g) = wk;
                if constexpr (WANT_DV) *(u32x4_t *)(vrow_out + 32 * cb + 16 * h + 8 * g) = wv;
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
    const long long BH = (long long)a.B * a.H;
    const int Npad = (a.N + kTile - 1) / kTile * kTile;
    float *L2 = static_cast<float *>(a.workspace);
    float *Dd = L2 + BH * Npad;
    const int xcd = (BH % 8 == 0) ? 1 : 0;
    const float c = a.scale * kLog2e;
    if (a.N > 0) {
        const long long prows = BH * Npad;
        const long long blocks = (prows * (D / 8) + kThreads - 1) / kThreads;
        hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           (const uint16_t *)a.O, (const uint16_t *)a.dO, a.LSE, L2, Dd, BH, a.N, Npad);
        const int n_qt = (a.N + kBq - 1) / kBq;
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(BH * n_qt)), dim3(kThreads), 0,
                           stream, (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (const uint16_t *)a.dO, (uint16_t *)a.dQ, L2, Dd, a.key_lens, a.H, a.N,
                           a.Nk, Npad, n_qt, xcd, c, a.scale);
    }
    if (a.Nk > 0) {
        const int n_kt = (a.Nk + kBk - 1) / kBk;
        auto dkdv = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)(BH * n_kt)), dim3(kThreads), 0, stream,
                               (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                               (const uint16_t *)a.dO, (uint16_t *)a.dK, (uint16_t *)a.dV, L2, Dd,
                               a.key_lens, a.H, a.N, a.Nk, Npad, n_kt, xcd, c, a.scale);
        };
        if constexpr (D == 64) {
            dkdv(bwd_dkdv_kernel<D, CAUSAL, kBoth>);
        } else {
            dkdv(bwd_dkdv_kernel<D, CAUSAL, kOnlyDV>);
            dkdv(bwd_dkdv_kernel<D, CAUSAL, kOnlyDK>);
        }
    }
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(long long B, long long H, long long N) {
    const long long npad = (N + kTile - 1) / kTile * kTile;
    return (size_t)(2 * B * H * npad) * sizeof(float);
}

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream) {
    if (a.d == 64) return a.causal ? launch_bwd<64, true>(a, stream) : launch_bwd<64, false>(a, stream);
    return a.causal ? launch_bwd<128, true>(a, stream) : launch_bwd<128, false>(a, stream);
}

}  // namespace fa
