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
// Two kernels, no atomics:
//   bwd_dq_kernel     one workgroup per 128 queries streams the K/V tiles (the
//                     forward's shape): S^T = K Q^T and dP^T = V dO^T with the
//                     query in the lane, then dQ^T += K^T dS^T with the K^T
//                     operand from the LDS transpose read.  It also computes
//                     D_i and LSE_i in log2 units (0 for a row with no key) and
//                     writes them for the second kernel.
//   bwd_dkdv_kernel   one workgroup per 128 keys (K and V fragments stay in
//                     VGPRs) streams the Q/dO tiles: S = Q K^T and dP = dO V^T
//                     with the key in the lane; reading the Q/dO rows in perm32
//                     order makes P and dS the B operand of dV^T += dO^T P and
//                     dK^T += Q^T dS directly, dO^T and Q^T come from transpose
//                     reads, and each lane ends with 16-byte pieces of its key's
//                     dK and dV rows.  At d = 128 (bwd_dkdv_paired_kernel) two
//                     waves share each 32 keys: one makes S, P and dV and hands
//                     P (bf16, its dV operand) to the other, which makes dP, dS
//                     and dK.
// Masking follows the forward exactly: causal key j <= i + (Nk - N), keys at
// or past key_lens[b] invisible; invisible pairs get P = 0, hence dS = 0.
// Both streaming kernels load their tiles from HBM straight into LDS (buffer
// loads with the LDS flag, one tile ahead, two stages held in separate arrays)
// and pipeline each tile by halves: the MFMAs that produce S and dP of the
// second 32-row block run beside the exponentials of the first, and the
// gradient MFMAs of the first block beside the exponentials of the second;
// that last phase issues at raised wave priority (s_setprio 1: 5% at d = 64,
// neutral at d = 128).
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
template <int N_> struct IntC { static constexpr int value = N_; };

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// Two floats to two fp16 (round to nearest even, v_cvt_pk_f16_f32), packed lo|hi.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}

template <int D> constexpr int kRowElems = D == 64 ? D + 8 : D + 24;
template <int D>
__device__ __forceinline__ int lds_at(int row, int col) { return row * kRowElems<D> + col; }

// dQ: 4 waves x 32 queries, K/V tiles of 64 keys through two LDS stages.
// KSPLIT = 2 (grids of at most one query block per CU): two groups of four
// waves share the block, group g taking the g-th half of its key tiles with
// its own stages; the partial dQ sums are added through LDS at the end.
template <int D, bool CAUSAL, int KSPLIT>
__global__ __launch_bounds__(kThreads * KSPLIT, KSPLIT > 1 ? 1 : 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ O, const uint16_t *__restrict__ dO,
    const float *__restrict__ LSE, uint16_t *__restrict__ dQ, float *__restrict__ L2,
    float *__restrict__ Dd, const int32_t *__restrict__ key_lens, int H, int N, int Nk, int Npad,
    int n_qtiles, int order, float c, float scale) {
    constexpr int TILE = kTile * kRowElems<D>;
    constexpr int KK = D / 16;
    constexpr int CB = D / 32;

    // one array per stage: the stage being loaded and the stage being read
    // are distinct objects, so no LDS read waits for the loads in flight
    static_assert(KSPLIT == 1 || KSPLIT == 2, "one or two key groups");
    __shared__ __attribute__((aligned(1024))) uint16_t Ks0[KSPLIT * TILE], Ks1[KSPLIT * TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs0[KSPLIT * TILE], Vs1[KSPLIT * TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave_id >= 0 && wave_id < kWaves * KSPLIT);
    const int grp = wave_id >> 2;               // key-split group
    const int wave = wave_id & (kWaves - 1);    // wave within the group: its 32 query rows
    const int li = lane & 31, g = lane >> 5;
    const int krow = perm32(li);
    // K^T operand through the transpose read (the forward's V^T read): lane li
    // receives K column perm32(li) of 4 consecutive keys per read
    const int trow = (li & 15) >> 2;
    const int tcol = perm32(4 * ((li & 3) + 4 * (li >> 4)));
    auto kst = [&](int stage) -> uint16_t * { return (stage ? Ks1 : Ks0) + grp * TILE; };
    auto vst = [&](int stage) -> uint16_t * { return (stage ? Vs1 : Vs0) + grp * TILE; };

    int bh, rank;
    block_in_order(blockIdx.x, gridDim.x / n_qtiles, n_qtiles, order, H, key_lens, Nk, bh, rank);
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
    // the group's key tiles: tbase .. tbase + half - 1 (those past ntiles only
    // join the barriers)
    const int half = (ntiles + KSPLIT - 1) / KSPLIT;
    const int tbase = grp * half;
    const int wq_first = q0 + wave * 32;
    const int wq_last = min(wq_first + 32, N) - 1;
    const int qrow = wq_first + li;

    const rsrc_t qsrc = make_rsrc(Q + q_base, (uint32_t)N * D * 2);
    const rsrc_t dosrc = make_rsrc(dO + q_base, (uint32_t)N * D * 2);

    // Q and dO fragments stay in VGPRs; O is read once for D_i = dO_i . O_i
    // (bf16 products exact in fp32, summed in fp32; lanes li and li + 32 hold
    // the two halves of each 16-column chunk)
    const rsrc_t osrc = make_rsrc(O + q_base, (uint32_t)N * D * 2);
    u32x4_t qf[KK], dof[KK];
    float dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const uint32_t ob = (uint32_t)(qrow * D + 16 * kk + 8 * g) * 2;
        qf[kk] = buffer_load16(qsrc, ob);
        dof[kk] = buffer_load16(dosrc, ob);
        const u32x4_t of = buffer_load16(osrc, ob);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t ow = of[w], gw = dof[kk][w];
            dpart = fmaf(bf16_bits_to_f32(ow & 0xffffu), bf16_bits_to_f32(gw & 0xffffu), dpart);
            dpart = fmaf(__builtin_bit_cast(float, ow & 0xffff0000u),
                         __builtin_bit_cast(float, gw & 0xffff0000u), dpart);
        }
    }
    const float dd = dpart + shfl_xor_f32(dpart, 32);
    // LSE in log2 units (0 when LSE = -inf: that row sees no key, so all of its
    // scores are masked anyway); a query past N takes l2 = +inf: every P of its
    // row is 0
    float l2 = __builtin_inff();
    if (qrow < N) {
        const float lse = LSE[(size_t)bh * N + qrow];
        l2 = lse == neg_inf() ? 0.f : lse * kLog2e;
    }
    // LSE2 and -D of the rows, for the dK/dV kernel that runs next (it starts
    // its dP accumulators at -D), in per-head arrays of Npad = N rounded up to
    // the 64-query tile; the padding gets zeros (its queries are masked there)
    if (grp == 0 && g == 0 && qrow < Npad) {
        L2[(size_t)bh * Npad + qrow] = qrow < N ? l2 : 0.f;
        Dd[(size_t)bh * Npad + qrow] = qrow < N ? -dd : 0.f;
    }
    wait_vmem_all();

    f32x16_t acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;

    // K/V tiles go from HBM straight into LDS: lane l of a wave's 16-byte
    // LDS load fills bytes 16 l .. 16 l + 15 of a 1 KiB window; a stage of
    // padded rows is NJ windows, wave w issues windows w, w + 4, ...  Each
    // lane's offset inside a tile is fixed (its window slot's row and 16-byte
    // column, or an out-of-range offset for the row padding: zeros).
    constexpr int RB = kRowElems<D> * 2;
    constexpr int NJ = kTile * RB / 1024, MJ = (NJ + kWaves - 1) / kWaves;
    static_assert(NJ * 1024 == kTile * RB, "stage is not a whole number of windows");
    uint32_t goff[MJ];
#pragma unroll
    for (int m = 0; m < MJ; ++m) {
        const int p = 1024 * (wave + kWaves * m) + 16 * lane;
        const int r = p / RB, q = (p % RB) / 16;
        goff[m] = (q < D / 8 && r < kTile) ? (uint32_t)(r * D * 2 + 16 * q) : 0x7ffffff0u;
    }
    auto refill = [&](int t, int stage) {
        const int j0 = t * kTile;
        const uint32_t bytes = (uint32_t)max(kv_end - j0, 0) * D * 2;
        const rsrc_t kr = make_rsrc(K + kv_base + (size_t)j0 * D, bytes);
        const rsrc_t vr = make_rsrc(V + kv_base + (size_t)j0 * D, bytes);
#pragma unroll
        for (int m = 0; m < MJ; ++m)
            if (wave + kWaves * m < NJ) {
                buffer_load_lds16(kr, (char *)kst(stage) + 1024 * (wave + kWaves * m), goff[m]);
                buffer_load_lds16(vr, (char *)vst(stage) + 1024 * (wave + kWaves * m), goff[m]);
            }
    };
    auto active = [&](int t) {
        return wq_first <= wq_last && (!CAUSAL || t * kTile <= wq_last + off);
    };
    // X^T = R F^T for one 32-key block jb of the tile: R rows (keys, perm32
    // order) from LDS, F the per-lane query fragment
    auto row_operand = [&](const uint16_t *R, int jb, int kk) {
        return *(const u32x4_t *)&R[lds_at<D>(32 * jb + krow, 16 * kk + 8 * g)];
    };
    auto rows_block = [&](const uint16_t *R, const u32x4_t (&F)[KK], int jb, f32x16_t &x) {
        x = mfma32(row_operand(R, jb, 0), F[0], f32x16_t{});
#pragma unroll
        for (int kk = 1; kk < KK; ++kk) x = mfma32(row_operand(R, jb, kk), F[kk], x);
    };
    auto kt_operand = [&](int stage, int cb, int jb, int h) {
        const auto *kb = (const __attribute__((address_space(3))) uint16_t *)kst(stage);
        const int r0 = 8 * g + trow + 32 * jb + 16 * h;
        const u32x2_t lo = lds_read_tr16(kb + lds_at<D>(r0, tcol + 32 * cb));
        const u32x2_t hi = lds_read_tr16(kb + lds_at<D>(r0 + 4, tcol + 32 * cb));
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };

    // tile t is read from stage t % 2 while tile t + 1 loads into the other;
    // unrolled by two so that both stages are compile-time objects
    auto tile = [&](auto par_c, int t) {
        constexpr int cur = decltype(par_c)::value;
        refill(t + 1, cur ^ 1);   // lands before this iteration's barrier
        if (t < ntiles && active(t)) {
            f32x16_t s[2], dp[2];
            uint32_t pk[2][8];
            const int j0 = t * kTile;
            const bool need_mask = (j0 + kTile > kv_lim) || (CAUSAL && j0 + kTile - 1 > wq_first + off);
            // P and dS of keys 2e, 2e + 1 of block jb, as the bf16 pair that
            // feeds dQ^T += K^T dS^T
            auto ds_pair = [&](int jb, int e) {
                const int v = 2 * e;
                const float p0 = exp2_hw(fmaf(s[jb][v], c, -l2));
                const float p1 = exp2_hw(fmaf(s[jb][v + 1], c, -l2));
                pk[jb][e] = pack_bf16x2(p0 * (dp[jb][v] - dd), p1 * (dp[jb][v + 1] - dd));
                pin(pk[jb][e]);
            };
            auto dq_mfma = [&](int cb, int jb, int h, const u32x4_t &kt) {
                acc[cb] = mfma32(kt, u32x4_t{pk[jb][4 * h], pk[jb][4 * h + 1], pk[jb][4 * h + 2], pk[jb][4 * h + 3]},
                                 acc[cb]);
            };
            // keys at or past this lane's limit are invisible; register v of block
            // jb holds key j0 + 32jb + 16(v/8) + 8g + v%8
            const int lim = (CAUSAL ? min(kv_lim, qrow + off + 1) : kv_lim) - j0 - 8 * g;
            auto mask_block = [&](int jb) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (32 * jb + 16 * (v >> 3) + (v & 7) >= lim) s[jb][v] = neg_inf();
            };
            // half-tile pipeline: the S, dP MFMAs of key block 1 run beside the
            // P, dS of block 0, and the dQ MFMAs of block 0 beside the P, dS of
            // block 1 (each accumulator sums in the same order as a plain loop)
            rows_block(kst(cur), qf, 0, s[0]);
            rows_block(vst(cur), dof, 0, dp[0]);
            if (need_mask) mask_block(0);
            constexpr int NB = 2 * KK;
            u32x4_t ra[2];
            ra[0] = row_operand(kst(cur), 1, 0);
            ra[1] = row_operand(vst(cur), 1, 0);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int kk = i >> 1;
                const u32x4_t a = ra[i & 1];
                if (i + 2 < NB) ra[i & 1] = row_operand((i & 1) ? vst(cur) : kst(cur), 1, kk + 1);
                if (i & 1) dp[1] = mfma32(a, dof[kk], kk == 0 ? f32x16_t{} : dp[1]);
                else s[1] = mfma32(a, qf[kk], kk == 0 ? f32x16_t{} : s[1]);
#pragma unroll
                for (int e = 8 * i / NB; e < 8 * (i + 1) / NB; ++e) ds_pair(0, e);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (need_mask) mask_block(1);
            // dQ MFMA i of a block adds half h = i / CB to accumulator i % CB:
            // consecutive MFMAs are independent, each accumulator adds its
            // halves in order
            constexpr int NQ = 2 * CB;
            __builtin_amdgcn_s_setprio(1);
            u32x4_t kt = kt_operand(cur, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const u32x4_t a = kt;
                if (i + 1 < NQ) kt = kt_operand(cur, (i + 1) % CB, 0, (i + 1) / CB);
                dq_mfma(i % CB, 0, i / CB, a);
#pragma unroll
                for (int e = 8 * i / NQ; e < 8 * (i + 1) / NQ; ++e) ds_pair(1, e);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int i = 0; i < NQ; ++i) dq_mfma(i % CB, 1, i / CB, kt_operand(cur, i % CB, 1, i / CB));
        }
        wait_vmem_all();
        __syncthreads();
    };
    refill(tbase, 0);
    wait_vmem_all();
    __syncthreads();
    int u = 0;   // the group's tile index
    for (; u + 2 <= half; u += 2) {
        tile(IntC<0>{}, tbase + u);
        tile(IntC<1>{}, tbase + u + 1);
    }
    if (u < half) tile(IntC<0>{}, tbase + u);

    if constexpr (KSPLIT > 1) {
        // group 1 hands its partial dQ to group 0 through the V stages (every
        // wave is past its last LDS read, no load in flight): one 256-byte row
        // per accumulator register, lane-indexed; group 0 adds it
        constexpr int RW = 16 * CB;
        constexpr int R0 = (int)(sizeof(Vs0) / 256);
        static_assert(kWaves * RW <= 2 * R0, "partial dQ does not fit the V stages");
        auto mrow = [&](int k) -> float * {
            const int r = wave * RW + k;
            return (r < R0 ? (float *)Vs0 + 64 * r : (float *)Vs1 + 64 * (r - R0)) + lane;
        };
        if (grp == 1) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int v = 0; v < 16; ++v) *mrow(16 * cb + v) = acc[cb][v];
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[cb][v] += *mrow(16 * cb + v);
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

// dK, dV at d = 64 (d = 128: bwd_dkdv_paired_kernel below): 4 waves x 32 keys;
// Q/dO tiles of 64 queries through two LDS stages.  KSPLIT = 2 (grids of at
// most one key block per CU): two groups of four waves share the block, group
// g taking the g-th half of its query tiles with its own stages; the partial
// sums are added through LDS.
template <int D, bool CAUSAL, int KSPLIT>
__global__ __launch_bounds__(kThreads * KSPLIT, KSPLIT > 1 ? 1 : 2) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, const float *__restrict__ L2, const float *__restrict__ Dd,
    const int32_t *__restrict__ key_lens, int H, int N, int Nk, int Npad, int n_ktiles,
    int order, float c, float scale) {
    constexpr int TILE = kTile * kRowElems<D>;
    constexpr int KK = D / 16;
    constexpr int CB = D / 32;
    static_assert(D == 64, "both accumulators beside the operands fit at d = 64 only");

    // one array per stage (see the dQ kernel); LD holds the tile's 64 LSE2
    // values followed by its 64 D values
    static_assert(KSPLIT == 1 || KSPLIT == 2, "one or two query groups");
    __shared__ __attribute__((aligned(1024))) uint16_t Qs0[KSPLIT * TILE], Qs1[KSPLIT * TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Gs0[KSPLIT * TILE], Gs1[KSPLIT * TILE];   // dO
    __shared__ __attribute__((aligned(16))) float LD0[KSPLIT * 2 * kTile], LD1[KSPLIT * 2 * kTile];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave_id >= 0 && wave_id < kWaves * KSPLIT);
    const int grp = wave_id >> 2;               // query-split group
    const int wave = wave_id & (kWaves - 1);    // wave within the group: its 32 keys
    const int li = lane & 31, g = lane >> 5;
    const int qperm = perm32(li);
    const int trow = (li & 15) >> 2;
    const int tcol = perm32(4 * ((li & 3) + 4 * (li >> 4)));
    auto qst = [&](int stage) -> uint16_t * { return (stage ? Qs1 : Qs0) + grp * TILE; };
    auto gst = [&](int stage) -> uint16_t * { return (stage ? Gs1 : Gs0) + grp * TILE; };
    auto ldst = [&](int stage) -> float * { return (stage ? LD1 : LD0) + grp * 2 * kTile; };

    int bh, rank;
    block_in_order(blockIdx.x, gridDim.x / n_ktiles, n_ktiles, order, H, key_lens, Nk, bh, rank);
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
    // the group's query tiles: tbase .. tbase + half - 1 (those past ntiles
    // only join the barriers)
    const int half = (ntiles + KSPLIT - 1) / KSPLIT;
    const int tbase = grp * half;

    const rsrc_t ksrc = make_rsrc(K + kv_base, (uint32_t)Nk * D * 2);
    const rsrc_t vsrc = make_rsrc(V + kv_base, (uint32_t)Nk * D * 2);
    // whole tiles of the padded per-head arrays: every 16-byte load is in range
    // or (prefetch past the last tile) entirely out of it
    const rsrc_t lsrc = make_rsrc(L2 + (size_t)bh * Npad, (uint32_t)Npad * 4);
    const rsrc_t dsrc = make_rsrc(Dd + (size_t)bh * Npad, (uint32_t)Npad * 4);

    u32x4_t kf[KK], vf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        kf[kk] = buffer_load16(ksrc, (uint32_t)(key * D + 16 * kk + 8 * g) * 2);
        vf[kk] = buffer_load16(vsrc, (uint32_t)(key * D + 16 * kk + 8 * g) * 2);
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

    // Q/dO tiles go from HBM straight into LDS (as the K/V tiles of the dQ
    // kernel); the tile's LSE2 and D values follow with one 16-lane load each
    // (waves 0 and 1), into LD[0..63] and LD[64..127]
    constexpr int RB = kRowElems<D> * 2;
    constexpr int NJ = kTile * RB / 1024, MJ = (NJ + kWaves - 1) / kWaves;
    static_assert(NJ * 1024 == kTile * RB, "stage is not a whole number of windows");
    uint32_t goff[MJ];
#pragma unroll
    for (int m = 0; m < MJ; ++m) {
        const int p = 1024 * (wave + kWaves * m) + 16 * lane;
        const int r = p / RB, q = (p % RB) / 16;
        goff[m] = (q < D / 8 && r < kTile) ? (uint32_t)(r * D * 2 + 16 * q) : 0x7ffffff0u;
    }
    auto refill = [&](int t, int stage) {
        const int i0 = (t_first + t) * kTile;
        const uint32_t bytes = (uint32_t)max(N - i0, 0) * D * 2;
        const rsrc_t qr = make_rsrc(Q + q_base + (size_t)i0 * D, bytes);
        const rsrc_t gr = make_rsrc(dO + q_base + (size_t)i0 * D, bytes);
#pragma unroll
        for (int m = 0; m < MJ; ++m)
            if (wave + kWaves * m < NJ) {
                buffer_load_lds16(qr, (char *)qst(stage) + 1024 * (wave + kWaves * m), goff[m]);
                buffer_load_lds16(gr, (char *)gst(stage) + 1024 * (wave + kWaves * m), goff[m]);
            }
        if (wave < 2 && lane < 16)
            buffer_load_lds16(wave == 0 ? lsrc : dsrc, (char *)ldst(stage) + 256 * wave, (uint32_t)(i0 + 4 * lane) * 4);
    };
    // a wave works on a tile if a query of it sees this wave's first key
    auto active = [&](int t) {
        const int i_last = (t_first + t) * kTile + kTile - 1;
        return wk0 < kv_lim && (!CAUSAL || i_last + off >= wk0);
    };
    // X = R F^T for the 32-query block qb of the tile (rows in perm32 order)
    // against this lane's key fragment F
    auto row_operand = [&](const uint16_t *R, int qb, int kk) {
        return *(const u32x4_t *)&R[lds_at<D>(32 * qb + qperm, 16 * kk + 8 * g)];
    };
    auto rows_block = [&](const uint16_t *R, const u32x4_t (&F)[KK], int qb, f32x16_t &x) {
        x = mfma32(row_operand(R, qb, 0), F[0], f32x16_t{});
#pragma unroll
        for (int kk = 1; kk < KK; ++kk) x = mfma32(row_operand(R, qb, kk), F[kk], x);
    };
    // transpose read of a Q or dO tile: lane li gets column 32cb + perm32(li)
    // of queries 32qb + 16h + 8g + 0..7
    auto t_operand = [&](const uint16_t *T, int cb, int qb, int h) {
        const auto *tb = (const __attribute__((address_space(3))) uint16_t *)T;
        const int r0 = 8 * g + trow + 32 * qb + 16 * h;
        const u32x2_t lo = lds_read_tr16(tb + lds_at<D>(r0, tcol + 32 * cb));
        const u32x2_t hi = lds_read_tr16(tb + lds_at<D>(r0 + 4, tcol + 32 * cb));
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };

    // tile t is read from stage t % 2 while tile t + 1 loads into the other;
    // within a tile the two 32-query blocks are software-pipelined as in the
    // dQ kernel: the S, dP MFMAs of block 1 run beside the P, dS of block 0,
    // the dV, dK MFMAs of block 0 beside the P, dS of block 1
    auto tile = [&](auto par_c, int t) {
        constexpr int cur = decltype(par_c)::value;
        refill(t + 1, cur ^ 1);   // lands before this iteration's barrier
        if (t < ntiles && active(t)) {
            const int i0 = (t_first + t) * kTile;
            const uint16_t *Qc = qst(cur), *Gc = gst(cur);
            const float *LDc = ldst(cur);
            f32x16_t s[2], dp[2];
            uint32_t pp[2][8], pd[2][8];
            // register v of block qb holds query i0 + 32qb + 16(v/8) + 8g + v%8
            const bool need_mask = !key_vis || (i0 + kTile > N) || (CAUSAL && i0 + off < wk0 + 31);
            auto mask_block = [&](int qb) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int i = i0 + 32 * qb + 16 * (v >> 3) + 8 * g + (v & 7);
                    if (!key_vis || i >= N || (CAUSAL && key > i + off)) s[qb][v] = neg_inf();
                }
            };
            // LSE2 of the 16 queries block qb gives this lane, and their -D as
            // the starting value of the block's dP accumulator (register order)
            f32x4_t lv[4];
            auto load_l = [&](int qb) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i8 = 32 * qb + 16 * h + 8 * g;
                    lv[2 * h] = *(const f32x4_t *)&LDc[i8];
                    lv[2 * h + 1] = *(const f32x4_t *)&LDc[i8 + 4];
                }
            };
            auto minus_d = [&](int qb) {
                f32x16_t x;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i8 = 32 * qb + 16 * h + 8 * g;
                    const f32x4_t a = *(const f32x4_t *)&LDc[kTile + i8];
                    const f32x4_t b = *(const f32x4_t *)&LDc[kTile + i8 + 4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[8 * h + e] = a[e];
                        x[8 * h + 4 + e] = b[e];
                    }
                }
                return x;
            };
            // P and dS of queries 2e, 2e + 1 of block qb as bf16 pairs
            auto p_pair = [&](int qb, int e) {
                const int v = 2 * e;
                const float l0 = lv[e >> 1][v & 3], l1 = lv[e >> 1][(v & 3) + 1];
                const float p0 = exp2_hw(fmaf(s[qb][v], c, -l0));
                const float p1 = exp2_hw(fmaf(s[qb][v + 1], c, -l1));
                pp[qb][e] = pack_bf16x2(p0, p1);
                pin(pp[qb][e]);
                pd[qb][e] = pack_bf16x2(p0 * dp[qb][v], p1 * dp[qb][v + 1]);   // dP - D
                pin(pd[qb][e]);
            };
            auto grad_mfma = [&](int cb, int qb, int h) {
                adv[cb] = mfma32(t_operand(Gc, cb, qb, h),
                                 u32x4_t{pp[qb][4 * h], pp[qb][4 * h + 1], pp[qb][4 * h + 2], pp[qb][4 * h + 3]},
                                 adv[cb]);
                adk[cb] = mfma32(t_operand(Qc, cb, qb, h),
                                 u32x4_t{pd[qb][4 * h], pd[qb][4 * h + 1], pd[qb][4 * h + 2], pd[qb][4 * h + 3]},
                                 adk[cb]);
            };
            rows_block(Qc, kf, 0, s[0]);
            dp[0] = minus_d(0);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) dp[0] = mfma32(row_operand(Gc, 0, kk), vf[kk], dp[0]);
            if (need_mask) mask_block(0);
            load_l(0);
            dp[1] = minus_d(1);
            // S and dP MFMAs of block 1, two P pairs of block 0 per S step
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                s[1] = mfma32(row_operand(Qc, 1, kk), kf[kk], kk == 0 ? f32x16_t{} : s[1]);
                dp[1] = mfma32(row_operand(Gc, 1, kk), vf[kk], dp[1]);
#pragma unroll
                for (int e = 8 * kk / KK; e < 8 * (kk + 1) / KK; ++e) p_pair(0, e);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (need_mask) mask_block(1);
            load_l(1);
            // dV, dK MFMAs of block 0 beside the P pairs of block 1
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < 2 * CB; ++i) {
                grad_mfma(i % CB, 0, i / CB);
#pragma unroll
                for (int e = 8 * i / (2 * CB); e < 8 * (i + 1) / (2 * CB); ++e) p_pair(1, e);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int i = 0; i < 2 * CB; ++i) grad_mfma(i % CB, 1, i / CB);
        }
        wait_vmem_all();
        __syncthreads();
    };
    refill(tbase, 0);
    wait_vmem_all();
    __syncthreads();
    int u = 0;   // the group's tile index
    for (; u + 2 <= half; u += 2) {
        tile(IntC<0>{}, tbase + u);
        tile(IntC<1>{}, tbase + u + 1);
    }
    if (u < half) tile(IntC<0>{}, tbase + u);

    if constexpr (KSPLIT > 1) {
        // group 1 hands its partial sums to group 0 through the Q and dO stages
        // (every wave is past its last LDS read, no load in flight): one
        // 256-byte row per accumulator register, lane-indexed
        constexpr int RW = 2 * 16 * CB;
        constexpr int R0 = (int)(sizeof(Qs0) / 256);
        static_assert(kWaves * RW <= 4 * R0, "partial sums do not fit the stages");
        auto mrow = [&](int k) -> float * {
            const int r = wave * RW + k, a = r / R0, rr = r - a * R0;
            uint16_t *base = a == 0 ? Qs0 : a == 1 ? Qs1 : a == 2 ? Gs0 : Gs1;
            return (float *)base + 64 * rr + lane;
        };
        // dK partials in rows 0 .. 16 CB - 1 of the wave's range, dV after them
        constexpr int VOFF = 16 * CB;
        if (grp == 1) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    *mrow(16 * cb + v) = adk[cb][v];
                    *mrow(VOFF + 16 * cb + v) = adv[cb][v];
                }
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                adk[cb][v] += *mrow(16 * cb + v);
                adv[cb][v] += *mrow(VOFF + 16 * cb + v);
            }
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
                *(u32x4_t *)(krow_out + 32 * cb + 16 * h + 8 * g) = wk;
                *(u32x4_t *)(vrow_out + 32 * cb + 16 * h + 8 * g) = wv;
            }
    }
}

// dK and dV of 128 keys in one pass (d = 128, where one wave cannot hold
// both accumulators beside its operands): 8 waves, waves w and w + 4 take the
// same 32 keys 32w .. 32w + 31 of the workgroup's 128 and share a SIMD.  Wave
// w (P side) keeps the K fragment: S = Q K^T, P = 2^(s c - LSE2) and
// dV^T += dO^T P; it hands P to wave w + 4 through LDS as fp16 pairs (P lies
// in [0, 1], where fp16 keeps 11 significant bits).  Wave w + 4 (dS side) keeps the V fragment and runs
// one Q/dO tile behind: dP - D = dO V^T - D, dS = P (dP - D) and
// dK^T += Q^T dS.  Iteration t: the P side works on tile t, the dS side on
// tile t - 1, tile t + 1 loads (three Q/dO stages).  P goes through two LDS
// buffers chosen by tile parity, so one barrier per iteration suffices: the
// P side makes S and P of tile t, stores P into buffer t mod 2 and adds dV;
// the dS side reads P(t - 1) from the other buffer, makes dP and dS and adds
// dK; the barrier at the end publishes P(t) and the loaded tile and puts
// every read of a buffer before its next write.
// Each tile's S and P are made once and its Q/dO cross HBM once (a launch
// per gradient would make S twice and read Q and dO twice); each gradient
// accumulator adds its tiles' terms in tile order.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(2 * kThreads, 1) void bwd_dkdv_paired_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, const float *__restrict__ L2, const float *__restrict__ Dd,
    const int32_t *__restrict__ key_lens, int H, int N, int Nk, int Npad, int n_ktiles,
    int order, float c, float scale) {
    constexpr int TILE = kTile * kRowElems<D>;
    constexpr int KK = D / 16;
    constexpr int CB = D / 32;
    constexpr int NW = 2 * kWaves;

    // three stages, one array each (see the dQ kernel)
    __shared__ __attribute__((aligned(1024))) uint16_t Qs0[TILE], Qs1[TILE], Qs2[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t Gs0[TILE], Gs1[TILE], Gs2[TILE];   // dO
    __shared__ __attribute__((aligned(16))) float LD0[2 * kTile], LD1[2 * kTile], LD2[2 * kTile];
    // bf16 P of two tiles (tile parity), [parity][key group][32-query block]
    // [half][lane][4 pairs]: each half of a block is one 1 KiB row, written and
    // read as 16 bytes per lane
    __shared__ __attribute__((aligned(1024))) uint32_t Pb[2 * kWaves * 2 * 2 * 64 * 4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave_id >= 0 && wave_id < NW);
    const int side = wave_id >> 2;              // 0: S, P, dV; 1: dP, dS, dK
    const int wave = wave_id & (kWaves - 1);    // its 32 keys
    const int li = lane & 31, g = lane >> 5;
    const int qperm = perm32(li);
    const int trow = (li & 15) >> 2;
    const int tcol = perm32(4 * ((li & 3) + 4 * (li >> 4)));
    auto qst = [&](int st) -> uint16_t * { return st == 0 ? Qs0 : st == 1 ? Qs1 : Qs2; };
    auto gst = [&](int st) -> uint16_t * { return st == 0 ? Gs0 : st == 1 ? Gs1 : Gs2; };
    auto ldst = [&](int st) -> float * { return st == 0 ? LD0 : st == 1 ? LD1 : LD2; };

    int bh, rank;
    block_in_order(blockIdx.x, gridDim.x / n_ktiles, n_ktiles, order, H, key_lens, Nk, bh, rank);
    const int b = bh / H;
    const int off = Nk - N;
    const int kv_lim = visible_len(key_lens, b, Nk);
    const size_t q_base = (size_t)bh * N * D;
    const size_t kv_base = (size_t)bh * Nk * D;

    const int k0 = rank * kBk;
    const int wk0 = k0 + wave * 32;
    const int key = wk0 + li;
    const bool key_vis = key < kv_lim;
    const int i_first = CAUSAL ? max(0, k0 - off) : 0;
    const int t_first = k0 < kv_lim ? i_first / kTile : 0;
    const int n_q = (N + kTile - 1) / kTile;
    const int ntiles = (k0 < kv_lim && i_first < N) ? n_q - t_first : 0;

    const rsrc_t lsrc = make_rsrc(L2 + (size_t)bh * Npad, (uint32_t)Npad * 4);
    const rsrc_t dsrc = make_rsrc(Dd + (size_t)bh * Npad, (uint32_t)Npad * 4);
    // the side's fragment of its keys: K (P side) or V (dS side)
    const rsrc_t fsrc = make_rsrc((side == 0 ? K : V) + kv_base, (uint32_t)Nk * D * 2);
    u32x4_t fr[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) fr[kk] = buffer_load16(fsrc, (uint32_t)(key * D + 16 * kk + 8 * g) * 2);
    f32x16_t ag[CB];   // dV (P side) or dK (dS side)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) ag[cb][v] = 0.f;

    // Q/dO tiles straight into LDS, the 1 KiB windows spread over all 8 waves:
    // load j of a wave is Q window j / 2 (j even) or dO window j / 2 (j odd),
    // load 2 MJ the tile's 64 LSE2 (wave 0) or D (wave 1) values
    constexpr int RB = kRowElems<D> * 2;
    constexpr int NJ = kTile * RB / 1024, MJ = (NJ + NW - 1) / NW, NL = 2 * MJ + 1;
    static_assert(NJ * 1024 == kTile * RB, "stage is not a whole number of windows");
    static_assert(NL <= 2 * KK, "loads outnumber the MFMA slots they are spread over");
    uint32_t goff[MJ];
#pragma unroll
    for (int m = 0; m < MJ; ++m) {
        const int p = 1024 * (wave_id + NW * m) + 16 * lane;
        const int r = p / RB, q = (p % RB) / 16;
        goff[m] = (q < D / 8 && r < kTile) ? (uint32_t)(r * D * 2 + 16 * q) : 0x7ffffff0u;
    }
    // the Q and dO ranges of tile t (whole tiles of the padded LSE2/D arrays)
    auto tile_src = [&](int t, rsrc_t &qr, rsrc_t &gr) {
        const int i0 = (t_first + t) * kTile;
        const uint32_t bytes = (uint32_t)max(N - i0, 0) * D * 2;
        qr = make_rsrc(Q + q_base + (size_t)i0 * D, bytes);
        gr = make_rsrc(dO + q_base + (size_t)i0 * D, bytes);
    };
    auto load_one = [&](int j, int t, int st, const rsrc_t &qr, const rsrc_t &gr) {
        const int i0 = (t_first + t) * kTile;
        if (j < 2 * MJ) {
            const int m = j >> 1;
            if (wave_id + NW * m < NJ)
                buffer_load_lds16(j & 1 ? gr : qr, (char *)(j & 1 ? gst(st) : qst(st)) + 1024 * (wave_id + NW * m),
                                  goff[m]);
        } else if (wave_id < 2 && lane < 16) {
            buffer_load_lds16(wave_id == 0 ? lsrc : dsrc, (char *)ldst(st) + 256 * wave_id,
                              (uint32_t)(i0 + 4 * lane) * 4);
        }
    };
    auto active = [&](int t) {
        const int i_last = (t_first + t) * kTile + kTile - 1;
        return wk0 < kv_lim && (!CAUSAL || i_last + off >= wk0);
    };
    // Each lane's element offsets within a tile for the row and transpose
    // reads, and its float offset within Ps.  Every iteration takes a fresh copy
    // of the last (an empty asm redefines it), so the P addresses are formed in
    // the iteration rather than held in registers across the loop (held, they
    // pushed the kernel past 256 VGPRs).
    const int row_lane0 = lds_at<D>(qperm, 8 * g);
    const int tr_lane0 = lds_at<D>(8 * g + trow, tcol);
    const int pw_lane0 = wave * (2 * 2 * 256) + 4 * lane;
    int row_lane = row_lane0, tr_lane = tr_lane0, pw_lane = pw_lane0;
    auto row_operand = [&](const uint16_t *R, int qb, int kk) {
        return *(const u32x4_t *)&R[row_lane + lds_at<D>(32 * qb, 16 * kk)];
    };
    auto t_operand = [&](const uint16_t *T, int cb, int qb, int h) {
        const auto *tb = (const __attribute__((address_space(3))) uint16_t *)T + tr_lane;
        const int r0 = 32 * qb + 16 * h;
        const u32x2_t lo = lds_read_tr16(tb + lds_at<D>(r0, 32 * cb));
        const u32x2_t hi = lds_read_tr16(tb + lds_at<D>(r0 + 4, 32 * cb));
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };
    // n MFMAs, MFMA i taking the LDS operand op(i) read two MFMAs ahead, with
    // body(i, operand) issuing it and any other work beside it
    auto pipelined = [&](auto n_c, auto op, auto body) {
        constexpr int n = decltype(n_c)::value;
        u32x4_t ring[2];
        ring[0] = op(0);
        ring[1] = op(1);
#pragma unroll
        for (int i = 0; i < n; ++i) {
            const u32x4_t cur = ring[i & 1];
            if (i + 2 < n) ring[i & 1] = op(i + 2);
            body(i, cur);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // gradient MFMA i adds half h = (i / CB) % 2 of block i / (2 CB) to
    // accumulator i % CB: consecutive MFMAs are independent, and each
    // accumulator adds its four terms in block, half order
    auto grad_mfmas = [&](const uint16_t *T, const uint32_t (&pk)[2][8], auto extra) {
        pipelined(IntC<4 * CB>{}, [&](int i) { return t_operand(T, i % CB, i / (2 * CB), (i / CB) & 1); },
                  [&](int i, const u32x4_t &a) {
                      const int qb = i / (2 * CB), cb = i % CB, h = (i / CB) & 1;
                      ag[cb] = mfma32(a, u32x4_t{pk[qb][4 * h], pk[qb][4 * h + 1], pk[qb][4 * h + 2], pk[qb][4 * h + 3]},
                                      ag[cb]);
                      extra(i);
                  });
    };

    // iteration t, stage of tile t: ST (compile time)
    auto iteration = [&](auto st_c, int t) {
        constexpr int ST = decltype(st_c)::value, ST_PREV = (ST + 2) % 3, ST_NEXT = (ST + 1) % 3;
        pw_lane = pw_lane0;
        asm volatile("" : "+v"(pw_lane));
        uint32_t *const pw = Pb + (t & 1) * (kWaves * 2 * 2 * 256) + pw_lane;         // P(t)
        const uint32_t *const pr = Pb + ((t + 1) & 1) * (kWaves * 2 * 2 * 256) + pw_lane;   // P(t - 1)
        const bool load_next = t + 1 < ntiles;
        rsrc_t qr, gr;
        tile_src(t + 1, qr, gr);
        auto issue = [&](int j) {
            if (load_next && j < NL) load_one(j, t + 1, ST_NEXT, qr, gr);
        };
        // S, then P (P side); dP - D, then dS (dS side); block qb in
        // x[qb], register v holding query i0 + 32qb + 16(v/8) + 8g + v%8
        f32x16_t x[2];
        uint32_t pk[2][8];
        const bool act0 = side == 0 && t < ntiles && active(t);
        const bool act1 = side == 1 && t >= 1 && active(t - 1);
        if (act0) {
            const int i0 = (t_first + t) * kTile;
            const uint16_t *Qc = qst(ST);
            const float *LDc = ldst(ST);
            pipelined(IntC<2 * KK>{}, [&](int i) { return row_operand(Qc, i & 1, i >> 1); },
                      [&](int i, const u32x4_t &a) {
                          const int qb = i & 1, kk = i >> 1;
                          x[qb] = mfma32(a, fr[kk], kk == 0 ? f32x16_t{} : x[qb]);
                          issue(i);
                      });
            if (!key_vis || (i0 + kTile > N) || (CAUSAL && i0 + off < wk0 + 31)) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int i = i0 + 32 * qb + 16 * (v >> 3) + 8 * g + (v & 7);
                        if (!key_vis || i >= N || (CAUSAL && key > i + off)) x[qb][v] = neg_inf();
                    }
            }
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                f32x4_t lv[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i8 = 32 * qb + 16 * h + 8 * g;
                    lv[2 * h] = *(const f32x4_t *)&LDc[i8];
                    lv[2 * h + 1] = *(const f32x4_t *)&LDc[i8 + 4];
                }
                // P of queries 2e, 2e + 1: a bf16 pair for dV, an fp16 pair
                // (P <= 1: eight times finer than bf16) for the dS side
                uint32_t ph[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int v = 2 * e;
                    const float p0 = exp2_hw(fmaf(x[qb][v], c, -lv[e >> 1][v & 3]));
                    const float p1 = exp2_hw(fmaf(x[qb][v + 1], c, -lv[e >> 1][(v & 3) + 1]));
                    pk[qb][e] = pack_bf16x2(p0, p1);
                    pin(pk[qb][e]);
                    ph[e] = pack_f16x2(p0, p1);
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    *(u32x4_t *)&pw[(2 * qb + hh) * 256] = u32x4_t{ph[4 * hh], ph[4 * hh + 1], ph[4 * hh + 2], ph[4 * hh + 3]};
            }
            grad_mfmas(gst(ST), pk, [](int) {});
        } else if (act1) {
            const float *LDc = ldst(ST_PREV);
            const uint16_t *Gc = gst(ST_PREV);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i8 = 32 * qb + 16 * h + 8 * g;
                    const f32x4_t a = *(const f32x4_t *)&LDc[kTile + i8];
                    const f32x4_t bb = *(const f32x4_t *)&LDc[kTile + i8 + 4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[qb][8 * h + e] = a[e];
                        x[qb][8 * h + 4 + e] = bb[e];
                    }
                }
            pipelined(IntC<2 * KK>{}, [&](int i) { return row_operand(Gc, i & 1, i >> 1); },
                      [&](int i, const u32x4_t &a) {
                          x[i & 1] = mfma32(a, fr[i >> 1], x[i & 1]);
                          issue(i);
                      });
            // dS from P(t - 1) (fp16 pairs), written by the P side before the last barrier
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const u32x4_t r = *(const u32x4_t *)&pr[(2 * qb + hh) * 256];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int e = 4 * hh + j, v = 2 * e;
                        const f16x2_t hv = __builtin_bit_cast(f16x2_t, (uint32_t)r[j]);
                        const float p0 = (float)hv[0], p1 = (float)hv[1];
                        pk[qb][e] = pack_bf16x2(p0 * x[qb][v], p1 * x[qb][v + 1]);
                        pin(pk[qb][e]);
                    }
                }
            grad_mfmas(qst(ST_PREV), pk, [](int) {});
        } else {
#pragma unroll
            for (int j = 0; j < NL; ++j) issue(j);
        }
        wait_vmem_all();
        __syncthreads();
    };
    if (ntiles > 0) {
        rsrc_t qr, gr;
        tile_src(0, qr, gr);
#pragma unroll
        for (int j = 0; j < NL; ++j) load_one(j, 0, 0, qr, gr);
    }
    wait_vmem_all();
    __syncthreads();
    const int nit = ntiles > 0 ? ntiles + 1 : 0;
    int t = 0;
    for (; t + 3 <= nit; t += 3) {
        iteration(IntC<0>{}, t);
        iteration(IntC<1>{}, t + 1);
        iteration(IntC<2>{}, t + 2);
    }
    if (t < nit) iteration(IntC<0>{}, t);
    if (t + 1 < nit) iteration(IntC<1>{}, t + 1);

    // accumulator register 8h + e of block cb holds d = 32cb + 16h + 8g + e of this lane's key
    if (key < Nk) {
        uint16_t *orow = (side == 0 ? dV : dK) + kv_base + (size_t)key * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4_t w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float a0 = ag[cb][8 * h + 2 * e], a1 = ag[cb][8 * h + 2 * e + 1];
                    if (side == 1) {
                        a0 *= scale;
                        a1 *= scale;
                    }
                    w[e] = pack_bf16x2(a0, a1);
                }
                *(u32x4_t *)(orow + 32 * cb + 16 * h + 8 * g) = w;
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
    const long long BH = (long long)a.B * a.H;
    const int Npad = (a.N + kTile - 1) / kTile * kTile;
    float *L2 = static_cast<float *>(a.workspace);
    float *Dd = L2 + BH * Npad;
    // the dQ kernel streams K and V of its head, the dK/dV kernel Q and dO.
    // The dK/dV kernel's Q/dO stream counts twice, so that the heads an XCD
    // runs at once keep it within half of the XCD's L2 (the other half takes
    // the gradients written back through it and the row statistics):
    // measured on B4 H16 N=2048 d=64 causal, its reads fall from 82.5 to
    // 68.4 MB (Q, K, V, dO once) and its time by 1%; counting the dQ
    // kernel's K/V stream twice as well cut its reads 93.6 -> 87.0 MB but
    // cost 3%.
    const int order_q = launch_order(a.B, a.H, CAUSAL, a.key_lens, 2ll * a.Nk * D * 2);
    const int order_k = launch_order(a.B, a.H, CAUSAL, a.key_lens, 2 * (2ll * a.N * D * 2));
    const float c = a.scale * kLog2e;
    if (a.N > 0) {
        // the dQ kernel also writes the D and LSE2 arrays the dK/dV kernel reads
        const int n_qt = (a.N + kBq - 1) / kBq;
        auto dq = [&](auto kern, int threads) {
            hipLaunchKernelGGL(kern, dim3((unsigned)(BH * n_qt)), dim3(threads), 0, stream,
                               (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                               (const uint16_t *)a.O, (const uint16_t *)a.dO, a.LSE, (uint16_t *)a.dQ,
                               L2, Dd, a.key_lens, a.H, a.N, a.Nk, Npad, n_qt, order_q, c, a.scale);
        };
        // at most one query block per CU: two key groups per block
        if (BH * n_qt <= device_cu_count()) dq(bwd_dq_kernel<D, CAUSAL, 2>, 2 * kThreads);
        else dq(bwd_dq_kernel<D, CAUSAL, 1>, kThreads);
    }
    if (a.Nk > 0) {
        const int n_kt = (a.Nk + kBk - 1) / kBk;
        auto dkdv = [&](auto kern, int threads) {
            hipLaunchKernelGGL(kern, dim3((unsigned)(BH * n_kt)), dim3(threads), 0, stream,
                               (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                               (const uint16_t *)a.dO, (uint16_t *)a.dK, (uint16_t *)a.dV, L2, Dd,
                               a.key_lens, a.H, a.N, a.Nk, Npad, n_kt, order_k, c, a.scale);
        };
        if constexpr (D == 64) {
            // at most one key block per CU: two query groups per block
            if (BH * n_kt <= device_cu_count()) dkdv(bwd_dkdv_kernel<D, CAUSAL, 2>, 2 * kThreads);
            else dkdv(bwd_dkdv_kernel<D, CAUSAL, 1>, kThreads);
        } else {
            // 8-wave workgroups at any grid size: measured faster than the two
            // query groups of the d = 64 kernel on grids of one block per CU
            dkdv(bwd_dkdv_paired_kernel<D, CAUSAL>, 2 * kThreads);
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
