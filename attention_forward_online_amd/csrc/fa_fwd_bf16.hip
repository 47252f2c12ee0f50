// fa_fwd_bf16.hip -- bf16 prefill attention forward on gfx950 matrix cores.
//
// Structure ('Online Softmax & FlashAttention' (interview lesson), Step 3):
// one workgroup owns a block of Br = 128 query rows for the whole loop
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
// gfx950 mapping (4 waves, 32 query rows per wave, 64-key tiles):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the Q fragment is the B
//     operand and stays in VGPRs for the whole loop; K rows come from LDS.
//     In the 32x32 accumulator each lane holds one query column, so a row
//     max/sum is an in-lane reduction plus one exchange with lane ^ 32
//     (v_permlane32_swap, no LDS traffic).
//   * The rows of each 32-key block are read in the order perm32 (bits 2 and
//     3 of the row index swapped).  Then accumulator registers 8h..8h+7 of
//     lane half g are keys 16h + 8g + 0..7: converted to bf16 they are the B
//     operand of O^T = V^T P^T without any data movement.
//   * K and V tiles are stored row-major in LDS alike; the V^T operand comes
//     from the gfx950 transpose read (ds_read_b64_tr_b16), two per MFMA.
//   * Scores stay fp32; exp runs as 2^(s*scale*log2 e - m'), one FMA plus
//     v_exp_f32 per score; P is rounded to bf16 (RNE) only as the MFMA operand
//     while the row sum uses the fp32 values.
//   * Lazy rescale: the reference max moves only when a tile's max exceeds it
//     by more than 2^8 (FA-4's thresholded rescale); o and l always share the
//     reference, so the result is unchanged while most tiles skip the
//     rescale of the accumulators.
//   * Work order: one query block per workgroup, causal launches start with
//     the longest blocks; all blocks of a head run on one XCD (the dispatcher
//     deals workgroup ids to the 8 XCDs round-robin), so K/V re-reads of a
//     head hit one L2, and consecutive heads go to different XCDs.  (Pairing
//     blocks n-1-u and u in one workgroup evens the work but halves the
//     waves per SIMD; it measured slower.)
//   * The MFMA sections run at raised wave priority (s_setprio 1), so the
//     arbiter issues a waiting wave's MFMAs ahead of the other wave's VALU
//     work and the matrix pipe stays fed.
//   * Two LDS stages, one barrier per tile: tile t is computed from one stage
//     while the other receives tile t+1 from registers; the global loads of
//     tile t+2 are in flight meanwhile.  Tiles are processed in order, with
//     the two waves of each SIMD (two workgroups per CU) overlapping one
//     wave's softmax with the other's MFMAs.  (Software-pipelining the next
//     tile's QK^T into the softmax within a wave measured slower on gfx950.)
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBc = 64;                     // keys per K/V tile
constexpr int kPad = 8;                     // bf16 pad per K/V row in LDS
constexpr float kLazyTau = 8.0f;            // log2 growth allowed before a rescale

// d = 64 fits three waves per SIMD (<= 168 VGPRs), d = 128 two.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 2) void fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE,
    const int32_t *__restrict__ key_lens, int H, int N, int Nk, int n_qtiles, int xcd_interleave,
    float c) {
    constexpr int NST = 2;                      // LDS stages
    constexpr int KS = D + kPad;                // K and V row stride in LDS (elements)
    constexpr int TILE = kBc * KS;              // elements per stage of K (or V)
    constexpr int KK = D / 16;                  // k-steps of S^T = K Q^T
    constexpr int CB = D / 32;                  // 32-column blocks of O^T
    constexpr int KCH = kBc * D / 8;            // 16-byte chunks per K (or V) tile
    constexpr int KL = KCH / kThreads;          // ... per thread
    static_assert(KCH % kThreads == 0, "tile/thread mismatch");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[NST * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[NST * TILE];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, g = lane >> 5;
    const int krow = perm32(li);
    // V^T operand through the transpose read: lane (li, g) reads the 4-element
    // chunk at key row vrow (+ the block's first key) and column vcol; lane li
    // then receives V column perm32(li) of 4 consecutive keys
    const int vrow = (li & 15) >> 2;
    const int vcol = perm32(4 * ((li & 3) + 4 * (li >> 4)));
    const __attribute__((address_space(3))) uint16_t *vs_lds =
        (const __attribute__((address_space(3))) uint16_t *)&Vs[0];

    // workgroup -> (head, query block).  With B*H divisible by 8, head bh lives on
    // XCD bh % 8 (the dispatcher deals workgroup ids to the XCDs round-robin):
    // all blocks of a head share one L2 and neighbouring heads spread over XCDs.
    const int BH = gridDim.x / n_qtiles;
    const int bid = blockIdx.x;
    int rank, bh;                   // rank: position of the block in launch order
    if (xcd_interleave) {
        const int hpx = BH >> 3, slot = bid >> 3;
        rank = slot / hpx;
        bh = (slot % hpx) * 8 + (bid & 7);
    } else {
        rank = bid / BH;
        bh = bid % BH;
    }
    const int b = bh / H;
    const int off = Nk - N;                     // causal: key j visible to query i iff j <= i + off
    const int kv_lim = visible_len(key_lens, b, Nk);
    const size_t q_base = (size_t)bh * N * D;
    const size_t kv_base = (size_t)bh * Nk * D;
    const rsrc_t qsrc = make_rsrc(Q + q_base, (uint32_t)N * D * 2);   // rows >= N read as 0

    // One query block per workgroup; causal launches hand out the longest
    // blocks (the last ones) first.
    {
        const int qtile = CAUSAL ? n_qtiles - 1 - rank : rank;
        const int q0 = qtile * kBr;
        int kv_end = kv_lim;
        if (CAUSAL) kv_end = min(kv_end, min(q0 + kBr, N) - 1 + off + 1);
        const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;
        const int wq_first = q0 + wave * kRowsPerWave;
        const int wq_last = min(wq_first + kRowsPerWave, N) - 1;   // < wq_first: no rows
        const int qrow = wq_first + li;
        const rsrc_t ksrc = make_rsrc(K + kv_base, (uint32_t)kv_end * D * 2);   // rows >= kv_end read as 0
        const rsrc_t vsrc = make_rsrc(V + kv_base, (uint32_t)kv_end * D * 2);

        u32x4_t qf[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[kk] = buffer_load16(qsrc, (uint32_t)(qrow * D + 16 * kk + 8 * g) * 2);
        // settle Q before the loop so that no wait inside it covers the prefetch
        wait_vmem_all();

        f32x16_t acc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
        // Reference max in log2 units (scale*log2(e)*score).  It moves only when
        // a tile's max exceeds it by more than kLazyTau (thresholded lazy
        // rescale, 'Online Softmax' research-hub page, "Why it matters"): the
        // weights 2^(s - ref) then stay below 2^kLazyTau, and o and l always
        // share one reference, so o / l and ref + log2 l are exact.
        float ms = neg_inf();
        float l = 0.f;          // this lane's half of the running denominator

        // Register stage for the global -> LDS copy.  Loads past the last tile
        // fall outside the buffer range and return zeros without touching
        // memory, so they are issued unconditionally (straight-line code keeps
        // the vmcnt waits partial).
        u32x4_t kr[KL], vr[KL];
        auto gload = [&](int t, u32x4_t (&kr)[KL], u32x4_t (&vr)[KL]) {
            const int j0 = t * kBc;
#pragma unroll
            for (int p = 0; p < KL; ++p) {
                const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
                const uint32_t off_b = (uint32_t)((j0 + row) * D + 8 * col8) * 2;
                kr[p] = buffer_load16(ksrc, off_b);
                vr[p] = buffer_load16(vsrc, off_b);
            }
        };
        auto lstore = [&](int stage, const u32x4_t (&kr)[KL], const u32x4_t (&vr)[KL]) {
#pragma unroll
            for (int p = 0; p < KL; ++p) {
                const int e = tid + kThreads * p, row = e / (D / 8), col8 = e % (D / 8);
                *(u32x4_t *)&Ks[stage * TILE + row * KS + 8 * col8] = kr[p];
                *(u32x4_t *)&Vs[stage * TILE + row * KS + 8 * col8] = vr[p];
            }
        };
        auto active = [&](int t) {   // wave-uniform; a prefix of the tiles
            return wq_first <= wq_last && (!CAUSAL || t * kBc <= wq_last + off);
        };
        // S^T of one 64-key tile (two 32-key blocks) x this wave's 32 queries,
        // operands read from LDS as the MFMAs need them
        auto qk_lds = [&](int stage, f32x16_t (&s)[2]) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const uint16_t *kp = &Ks[stage * TILE + (32 * jb + krow) * KS + 8 * g];
                s[jb] = mfma32(*(const u32x4_t *)kp, qf[0], f32x16_t{});
#pragma unroll
                for (int kk = 1; kk < KK; ++kk)
                    s[jb] = mfma32(*(const u32x4_t *)(kp + 16 * kk), qf[kk], s[jb]);
            }
        };
        // V^T operand (A of the P.V MFMA) for keys 32jb + 16h + 8g + 0..7 and
        // V column 32cb + perm32(li) of the tile in `stage`
        auto v_operand = [&](int stage, int cb, int jb, int h) {
            const auto *p0 =
                vs_lds + stage * TILE + (8 * g + vrow + 32 * jb + 16 * h) * KS + vcol + 32 * cb;
            const u32x2_t lo = lds_read_tr16(p0);
            const u32x2_t hi = lds_read_tr16(p0 + 4 * KS);
            return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        };
        // masking, row max and the (rare) move of the reference; returns the
        // reference the probabilities of this tile use
        auto softmax_prep = [&](int t, f32x16_t (&sc)[2]) {
            const int j0 = t * kBc;
            const bool need_mask =
                (j0 + kBc > kv_lim) || (CAUSAL && j0 + kBc - 1 > wq_first + off);
            if (need_mask) {
                // register v of block jb holds key j0 + 32jb + 16(v/8) + 8g + v%8;
                // keys at or past this lane's limit are invisible
                const int vis_end = CAUSAL ? min(kv_lim, qrow + off + 1) : kv_lim;
                const int lim = vis_end - j0 - 8 * g;
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (32 * jb + 16 * (v >> 3) + (v & 7) >= lim) sc[jb][v] = neg_inf();
            }
            // tile row max: four independent chains over the 32 in-lane keys,
            // the other 32 keys in lane ^ 32
            float m4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x16_t &s = sc[i >> 1];
                const int v0 = 8 * (i & 1);
                m4[i] = fmaxf(fmaxf(fmaxf(s[v0], s[v0 + 1]), s[v0 + 2]),
                              fmaxf(fmaxf(s[v0 + 3], s[v0 + 4]),
                                    fmaxf(fmaxf(s[v0 + 5], s[v0 + 6]), s[v0 + 7])));
            }
            const float mx = max_xor32(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * c;
            // move the reference only when this row's max got too far ahead
            const bool move = mx > ms + kLazyTau;   // false for a fully masked tile
            if (__any(move)) {
                // lanes that keep their reference use alpha = 1 (never
                // exp2(ms - ms), which is NaN while ms is still -inf)
                const float alpha = move ? exp2_hw(ms - mx) : 1.f;   // 0 when ms = -inf
                l *= alpha;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[cb][v] *= alpha;
                ms = move ? mx : ms;
            }
            return ms == neg_inf() ? 0.f : ms;   // -inf guard: all P = 0 then
        };
        // P = 2^(s c - ref) for this lane's 32 scores: bf16 pairs for the MFMA,
        // fp32 values into the row sum (four partial sums)
        auto probabilities = [&](const f32x16_t (&sc)[2], float ms_ref, uint32_t (&pk)[2][8]) {
            float r4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const float p0 = exp2_hw(fmaf(sc[jb][v], c, -ms_ref));
                    const float p1 = exp2_hw(fmaf(sc[jb][v + 1], c, -ms_ref));
                    r4[(v >> 1) & 3] += p0 + p1;
                    pk[jb][v >> 1] = pack_bf16x2(p0, p1);
                }
            return (r4[0] + r4[1]) + (r4[2] + r4[3]);
        };
        auto p_operand = [&](const uint32_t (&pk)[2][8], int jb, int h) {
            return u32x4_t{pk[jb][4 * h], pk[jb][4 * h + 1], pk[jb][4 * h + 2], pk[jb][4 * h + 3]};
        };

        // tiles in order from two LDS stages; the loads of tile t+1 are in
        // flight while tile t is computed
        gload(0, kr, vr);
        lstore(0, kr, vr);
        gload(1, kr, vr);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            const int cur = t & 1;
            if (active(t)) {
                f32x16_t sc[2];
                __builtin_amdgcn_s_setprio(1);
                qk_lds(cur, sc);
                __builtin_amdgcn_s_setprio(0);
                const float ms_ref = softmax_prep(t, sc);
                uint32_t pk[2][8];
                l += probabilities(sc, ms_ref, pk);
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            acc[cb] = mfma32(v_operand(cur, cb, jb, h), p_operand(pk, jb, h),
                                             acc[cb]);
                __builtin_amdgcn_s_setprio(0);
            }
            lstore(cur ^ 1, kr, vr);    // tile t+1
            gload(t + 2, kr, vr);
            __syncthreads();
        }

        // epilogue: O = o / l (0 for a row without keys), LSE = ref + log2 l in nats (-inf then)
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
                        w[e] = pack_bf16x2(acc[cb][8 * h + 2 * e] * inv,
                                           acc[cb][8 * h + 2 * e + 1] * inv);
                    *(u32x4_t *)(orow + 32 * cb + 16 * h + 8 * g) = w;
                }
            if (g == 0)
                LSE[(size_t)bh * N + qrow] = lt > 0.f ? (ms + log2_hw(lt)) * kLn2 : neg_inf();
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs &a, hipStream_t stream) {
    const int n_qtiles = (a.N + kBr - 1) / kBr;
    const long long BH = (long long)a.B * a.H;
    const long long nblocks = BH * n_qtiles;
    const int xcd_interleave = (BH % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)nblocks), dim3(kThreads), 0,
                       stream, (const uint16_t *)a.Q, (const uint16_t *)a.K,
                       (const uint16_t *)a.V, (uint16_t *)a.O, a.LSE, a.key_lens, a.H, a.N,
                       a.Nk, n_qtiles, xcd_interleave, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream) {
    if (a.d == 64) return a.causal ? launch_one<64, true>(a, stream) : launch_one<64, false>(a, stream);
    return a.causal ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
}

}  // namespace fa
