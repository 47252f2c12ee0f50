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
//   * K and V tiles are stored row-major in LDS; the V^T operand comes from
//     the gfx950 transpose read (ds_read_b64_tr_b16), two per MFMA.  The row
//     strides differ: a transpose read serves 32 lanes per pass, four rows of
//     16 banks each, and V's stride keeps those rows in disjoint banks (with
//     K's stride they collided 2-way at d = 64 and 4-way at d = 128).
//   * Scores stay fp32; exp runs as 2^(s*scale*log2 e - m'), one FMA plus
//     v_exp_f32 per score; P is rounded to bf16 (RNE) only as the MFMA operand
//     while the row sum uses the fp32 values.
//   * Conditional rescale (FA-4 on the research-hub 'Online Softmax' page,
//     "Why it matters": rescale only when the max shift threatens stability).
//     o and l always share one reference m', so o / l and m' + log2 l are
//     exact whatever m' is, as long as no weight 2^(s - m') overflows.  The
//     default rule (overflow guard) therefore takes no per-tile row max: each
//     group of weights is made against the current m', and only when some
//     lane's sum of a group reaches 2^32 (or a lane has no m' yet) is the
//     group's max taken, m' moved to it, o and l rescaled and the group made
//     again.  The first tile's max is always taken.  Two ablation rules keep
//     the per-tile max: the threshold rule (m' moves when the max grows by
//     more than 8 in log2 units) and the eager rule (every tile, the plain
//     recurrence).
//   * Software pipeline within each wave: iteration t issues the MFMAs of
//     S(t+1) = K(t+1) Q^T with the exponentials of tile t between them, then
//     the MFMAs of O += P(t) V(t) with the rest of those exponentials (and,
//     under the ablation rules, the row max of tile t+1) between them, so the
//     matrix pipe and the vector ALUs of one wave work at the same time.  The
//     guard checks each group of weights before the first MFMA that uses it.  Scheduling barriers fix the order of
//     each MFMA and its VALU group; pin() keeps the compiler from sinking the
//     VALU work towards its later uses.  The loop is unrolled by two so that
//     S(t) and S(t+1) alternate between two register sets without copies.
//   * K/V tiles go from HBM straight into LDS (buffer loads with the LDS flag,
//     no register stage), which keeps d = 64 within three waves per SIMD and
//     d = 128 without spills.  K runs two tiles ahead, V one: iteration t
//     loads K(t+2) into the stage K(t) left and V(t+1) into the stage V(t-1)
//     left, and they land before the iteration's only barrier.
//   * Small grids (at most one query block per CU): each block's
//     key tiles are split in two halves run by two groups of four waves in
//     one workgroup, each with its own LDS stages and its own (m, l, o); at
//     the end group 1 hands its state to group 0 through LDS and group 0
//     merges the two with the (m, l) merge ('Online Softmax & FlashAttention',
//     Step 1) before the epilogue.  Blocks without any visible key write
//     O = 0, LSE = -inf and leave at once.
//   * Work order: one query block per workgroup, causal launches start with
//     the longest blocks; all blocks of a head run on one XCD (the dispatcher
//     deals workgroup ids to the 8 XCDs round-robin), so K/V re-reads of a
//     head hit one L2, and consecutive heads go to different XCDs.
#include <atomic>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBc = 64;                     // keys per K/V tile
// LDS row strides (bf16 elements).  In 4-byte banks modulo 64: K rows step
// by 4 x odd banks, so the 16 rows one ds_read_b128 pass reads (16 lanes) start
// in distinct 4-bank groups; V rows step by 16 or 48 banks, so the four rows
// one pass of ds_read_b64_tr_b16 reads (32 lanes, 16 banks per row) fall in
// disjoint bank ranges.
constexpr int kPadK = 8;
constexpr int kPadV = 32;
constexpr float kLazyTau = 8.0f;            // log2 growth allowed before a rescale (threshold rule)
// Overflow-guard rule: a tile's weights, taken against the current reference,
// are kept when every lane's sum of them stays below 2^32 (so every weight is
// below 2^32 and, over at most 2^31 keys, l stays below 2^63: far inside fp32);
// otherwise the tile's max is taken and the reference moves to it.
constexpr float kGuardLimit = 4294967296.0f;
constexpr int kPrefetch = 2;                // LDS operands read this many MFMAs ahead

template <int N_> struct IntC { static constexpr int value = N_; };
template <bool B_> struct BoolC { static constexpr bool value = B_; };

// d = 64 fits three waves per SIMD (<= 168 VGPRs), d = 128 two.  KSPLIT = 2:
// two groups of four waves share each query block, group g taking the g-th
// half of its key tiles; their states are merged at the end.
template <int D, bool CAUSAL, int KSPLIT, int RULE>
__global__ __launch_bounds__(kThreads * KSPLIT, KSPLIT > 1 ? 1 : (D == 64 ? 3 : 2)) void fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE,
    const int32_t *__restrict__ key_lens, int H, int N, int Nk, int n_qtiles, int order,
    float c) {
    constexpr int KS = D + kPadK;               // K row stride in LDS (elements)
    constexpr int VS = D + kPadV;               // V row stride in LDS (elements)
    static_assert((KS / 2) % 8 == 4 && (VS / 2) % 32 == 16, "LDS strides off the bank pattern");
    constexpr int KK = D / 16;                  // k-steps of S^T = K Q^T
    constexpr int CB = D / 32;                  // 32-column blocks of O^T
    constexpr bool GUARD = RULE == kRuleGuard;
    constexpr int NS = 2 * KK;                  // S MFMAs per tile (= P pairs made beside them)
    constexpr int NP2 = 4 * CB;                 // P.V MFMAs per tile
    constexpr int PAIRS2 = 16 - NS;             // P pairs left for the P.V section
    constexpr int PD = kPrefetch;
    // the phase whose waves issue at raised priority (s_setprio 1): the P.V
    // phase at d = 64, the S phase at d = 128 (measured: 2-3% each, the other
    // choice neutral)
    constexpr int kPrioPhase = D == 64 ? 2 : 1;
    // the pairs beside the S MFMAs in a three-stage pipeline (d = 128: two
    // waves per SIMD at most, so a slot's dependent VALU chain is not hidden by
    // other waves); d = 64 keeps three waves per SIMD and one pair per slot
    constexpr bool kStagedPairs = D == 128;
    static_assert(PAIRS2 % 2 == 0 && PAIRS2 / 2 + 4 <= NP2, "P.V section too short");
    // the guard checks the pairs made beside the P.V MFMAs before the MFMAs
    // that use them: all of them are made beside the first half
    static_assert(PAIRS2 == 0 || (PAIRS2 / 2 == NP2 / 2 && NS / 4 == NP2 / (2 * CB)),
                  "guard: second pair group must end half way through P.V");
    static_assert(KSPLIT >= 1 && KSPLIT <= 3, "one to three key groups");

    // one array per stage, so that the stage a load fills and the stage the
    // MFMAs read are distinct objects (with a key split: one half per group)
    __shared__ __attribute__((aligned(1024))) uint16_t Ks0[KSPLIT * kBc * KS], Ks1[KSPLIT * kBc * KS];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs0[KSPLIT * kBc * VS], Vs1[KSPLIT * kBc * VS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave_id >= 0 && wave_id < kWaves * KSPLIT);
    const int grp = wave_id >> 2;               // key-split group
    const int wave = wave_id & (kWaves - 1);    // wave within the group: its 32 query rows
    const int li = lane & 31, g = lane >> 5;
    const int krow = perm32(li);
    const int vrow = (li & 15) >> 2;
    const int vcol = perm32(4 * ((li & 3) + 4 * (li >> 4)));
    auto kst = [&](int stage) -> uint16_t * { return (stage ? Ks1 : Ks0) + grp * (kBc * KS); };
    auto vst = [&](int stage) -> uint16_t * { return (stage ? Vs1 : Vs0) + grp * (kBc * VS); };

    // workgroup -> (head, query block) in the launch order `order`
    const int BH = gridDim.x / n_qtiles;
    const int bid = blockIdx.x;
    int rank, bh;                   // rank: position of the block in launch order
    block_in_order(bid, BH, n_qtiles, order, H, key_lens, Nk, bh, rank);
    const int b = bh / H;
    const int off = Nk - N;                     // causal: key j visible to query i iff j <= i + off
    const int kv_lim = __builtin_amdgcn_readfirstlane(visible_len(key_lens, b, Nk));
    const size_t q_base = (size_t)bh * N * D;
    const size_t kv_base = (size_t)bh * Nk * D;
    const rsrc_t qsrc = make_rsrc(Q + q_base, (uint32_t)N * D * 2);

    // causal launches hand out the longest blocks (the last ones) first
    const int qtile = CAUSAL ? n_qtiles - 1 - rank : rank;
    const int q0 = qtile * kBr;
    int kv_end = kv_lim;
    if (CAUSAL) kv_end = min(kv_end, min(q0 + kBr, N) - 1 + off + 1);
    const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;
    const int wq_first = q0 + wave * kRowsPerWave;
    const int wq_last = min(wq_first + kRowsPerWave, N) - 1;
    const int qrow = wq_first + li;
    if (ntiles == 0) {      // no visible key in the block: O = 0, LSE = -inf
        if (grp == 0 && qrow < N) {
            uint16_t *orow = O + q_base + (size_t)qrow * D;
#pragma unroll
            for (int j = 0; j < D / 16; ++j)
                *(u32x4_t *)(orow + 16 * j + 8 * g) = u32x4_t{0u, 0u, 0u, 0u};
            if (g == 0) LSE[(size_t)bh * N + qrow] = neg_inf();
        }
        return;
    }
    // the group's key tiles: tiles tbase .. tbase + ntg - 1 of the block; both
    // groups pass nloop barriers in the tile loop
    const int half = (ntiles + KSPLIT - 1) / KSPLIT;
    const int tbase = grp * half;
    const int ntg = min(max(ntiles - tbase, 0), half);
    const int nloop = half;
    // tiles this wave sees: a prefix of the block's tiles (all of them unless
    // causal), of which its group takes the part from tbase on
    int nt_w = 0;
    if (wq_first <= wq_last) {
        const int last_key = wq_last + off;
        const int seen = !CAUSAL ? ntiles : (last_key < 0 ? 0 : min(ntiles, last_key / kBc + 1));
        nt_w = min(max(seen - tbase, 0), ntg);
    }

    u32x4_t qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = buffer_load16(qsrc, (uint32_t)(qrow * D + 16 * kk + 8 * g) * 2);   // rows >= N read 0

    f32x16_t acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
    // Reference max in log2 units (scale*log2(e)*score), moved by the rescale
    // rule (RULE): the guard moves it only when a group's weights could reach
    // kGuardLimit, the threshold rule when a tile's max exceeds it by more
    // than kLazyTau, the eager rule on every tile.  o and l always share one
    // reference, so o / l and ref + log2 l are exact under every rule.
    float ms = neg_inf();
    float ref = 0.f;        // the reference the next probabilities use (0 while ms = -inf)
    float l = 0.f;          // this lane's half of the running denominator
    bool all_ref = false;   // guard rule: every lane of the wave has a finite reference

    // K/V tiles go from HBM straight into LDS (16-byte buffer loads with the
    // LDS flag: lane l of a wave's load fills bytes 16 l .. 16 l + 15 of a 1 KiB
    // window).  A stage of rows of RS elements is a whole number of such
    // windows; wave w issues windows w, w + 4, ...  Each lane's global offset
    // within the tile is fixed: its window position's row and 16-byte column,
    // or an offset past every buffer for the row padding (the range check then
    // writes zeros).
    auto window_offsets = [&](auto rs_c, uint32_t *goff) {
        constexpr int RB = decltype(rs_c)::value * 2;   // LDS row bytes
        constexpr int NJ = kBc * RB / 1024, MJ = (NJ + kWaves - 1) / kWaves;
#pragma unroll
        for (int m = 0; m < MJ; ++m) {
            const int p = 1024 * (wave + kWaves * m) + 16 * lane;
            const int r = p / RB, q = (p % RB) / 16;
            goff[m] = (q < D / 8 && r < kBc) ? (uint32_t)(r * D * 2 + 16 * q) : 0x7ffffff0u;
        }
    };
    constexpr int NJK = kBc * KS * 2 / 1024, NJV = kBc * VS * 2 / 1024;
    constexpr int MJK = (NJK + kWaves - 1) / kWaves, MJV = (NJV + kWaves - 1) / kWaves;
    static_assert(NJK * 1024 == kBc * KS * 2 && NJV * 1024 == kBc * VS * 2,
                  "stage is not a whole number of windows");
    uint32_t goffk[MJK], goffv[MJV];
    window_offsets(IntC<KS>{}, goffk);
    window_offsets(IntC<VS>{}, goffv);
    auto dma = [&](auto nj_c, const uint32_t *goff, const uint16_t *src, uint16_t *dst, int t) {
        constexpr int NJ = decltype(nj_c)::value, MJ = (NJ + kWaves - 1) / kWaves;
        const int j0 = (tbase + t) * kBc;
        const rsrc_t r = make_rsrc(src + (size_t)j0 * D, (uint32_t)max(kv_end - j0, 0) * D * 2);
#pragma unroll
        for (int m = 0; m < MJ; ++m)
            if (wave + kWaves * m < NJ)
                buffer_load_lds16(r, (char *)dst + 1024 * (wave + kWaves * m), goff[m]);
    };
    auto dma_k = [&](uint16_t *dst, int t) { dma(IntC<NJK>{}, goffk, K + kv_base, dst, t); };
    auto dma_v = [&](uint16_t *dst, int t) { dma(IntC<NJV>{}, goffv, V + kv_base, dst, t); };
    // Each lane's element offsets within a K and a V stage, computed once: the
    // operands below add only compile-time offsets to them.
    const int k_lane = krow * KS + 8 * g;
    const int v_lane = (8 * g + vrow) * VS + vcol;
    // operand of S MFMA i (block jb = i % 2, k-step kk = i / 2) from the K tile in `stage`
    auto k_operand = [&](int stage, int i) {
        const int jb = i & 1, kk = i >> 1;
        return *(const u32x4_t *)&kst(stage)[k_lane + 32 * jb * KS + 16 * kk];
    };
    // operand of P.V MFMA i (chunk ci = i / CB = 2 jb + h, column block cb = i % CB)
    auto v_operand = [&](int stage, int i) {
        const int ci = i / CB, cb = i % CB, jb = ci >> 1, h = ci & 1;
        const auto *p0 = (const __attribute__((address_space(3))) uint16_t *)vst(stage) + v_lane +
                         (32 * jb + 16 * h) * VS + 32 * cb;
        const u32x2_t lo = lds_read_tr16(p0);
        const u32x2_t hi = lds_read_tr16(p0 + 4 * VS);
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };
    // P pair q (chunk q / 4, scores 2(q % 4), +1 of it): 2^(s c - ref) in fp32 into the
    // row sum, bf16 pair into the MFMA operand
    auto p_pair = [&](const f32x16_t (&s)[2], int q, uint32_t (&pk)[4][4], float (&rs)[4]) {
        const int ci = q >> 2, e = q & 3, jb = ci >> 1, v = 8 * (ci & 1) + 2 * e;
        const float p0 = exp2_hw(fmaf(s[jb][v], c, -ref));
        const float p1 = exp2_hw(fmaf(s[jb][v + 1], c, -ref));
        rs[q & 3] += p0 + p1;
        pk[ci][e] = pack_bf16x2(p0, p1);
        pin(rs[q & 3]);
        pin(pk[ci][e]);
    };
    // The same pair in three stages for a software pipeline across MFMA slots
    // (slot i: arguments of pair i, exponentials of pair i - 1, sum and pack of
    // pair i - 2), so that no VALU instruction of a slot waits on another of
    // the same slot: the arithmetic and the rounding are those of p_pair.
    auto pair_args = [&](const f32x16_t (&s)[2], int q, float (&x)[2]) {
        const int ci = q >> 2, e = q & 3, jb = ci >> 1, v = 8 * (ci & 1) + 2 * e;
        x[0] = fmaf(s[jb][v], c, -ref);
        x[1] = fmaf(s[jb][v + 1], c, -ref);
        pin(x[0]);
        pin(x[1]);
    };
    auto pair_exp = [&](float (&x)[2]) {
        x[0] = exp2_hw(x[0]);
        x[1] = exp2_hw(x[1]);
        pin(x[0]);
        pin(x[1]);
    };
    auto pair_keep = [&](int q, const float (&p)[2], uint32_t (&pk)[4][4], float (&rs)[4]) {
        const int ci = q >> 2, e = q & 3;
        rs[q & 3] += p[0] + p[1];
        pk[ci][e] = pack_bf16x2(p[0], p[1]);
        pin(rs[q & 3]);
        pin(pk[ci][e]);
    };
    auto max8 = [&](const f32x16_t (&s)[2], int k) {
        const f32x16_t &x = s[k >> 1];
        const int v0 = 8 * (k & 1);
        return fmaxf(fmaxf(fmaxf(x[v0], x[v0 + 1]), x[v0 + 2]),
                     fmaxf(fmaxf(x[v0 + 3], x[v0 + 4]), fmaxf(fmaxf(x[v0 + 5], x[v0 + 6]), x[v0 + 7])));
    };
    auto need_mask = [&](int t) {
        const int j0 = (tbase + t) * kBc;
        return (j0 + kBc > kv_lim) || (CAUSAL && j0 + kBc - 1 > wq_first + off);
    };
    auto apply_mask = [&](int t, f32x16_t (&sc)[2]) {
        const int j0 = (tbase + t) * kBc;
        const int vis_end = CAUSAL ? min(kv_lim, qrow + off + 1) : kv_lim;
        const int lim = vis_end - j0 - 8 * g;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (32 * jb + 16 * (v >> 3) + (v & 7) >= lim) sc[jb][v] = neg_inf();
    };
    // move of the reference after a tile's row max mx (log2 units).  Eager:
    // every tile, m' = max(m', mx) and o, l *= 2^(m'_old - m') (the plain
    // recurrence).  Threshold: only lanes whose max grew by more than kLazyTau
    // move, and the accumulators are touched only when some lane of the wave
    // moves.  Guard: called on the slow path only, any growth moves.
    // Returns the factor o and l were scaled by (1 when nothing moved).
    auto decide = [&](float mx) {
        float alpha = 1.f;
        if constexpr (RULE == kRuleEager) {
            const float mn = fmaxf(ms, mx);
            alpha = mn == neg_inf() ? 1.f : exp2_hw(ms - mn);   // 0 when ms = -inf
            l *= alpha;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[cb][v] *= alpha;
            ms = mn;
        } else {
            const bool move = mx > ms + (RULE == kRuleTau ? kLazyTau : 0.f);   // false for a fully masked tile
            if (__any(move)) {
                alpha = move ? exp2_hw(ms - mx) : 1.f;   // 0 when ms = -inf
                l *= alpha;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[cb][v] *= alpha;
                ms = move ? mx : ms;
            }
        }
        ref = ms == neg_inf() ? 0.f : ms;
        if constexpr (GUARD) all_ref = !__any(ms == neg_inf());
        return alpha;
    };
    auto rowmax = [&](const float (&m4)[4]) {
        return max_xor32(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * c;
    };

    // prologue: K(0), V(0), K(1) into LDS, issued with the Q loads; S(0) is
    // prepared as soon as Q and K(0) have landed (every wave has at most its
    // V(0) and K(1) windows outstanding), the rest arrives meanwhile
    dma_k(kst(0), 0);
    dma_v(vst(0), 0);
    dma_k(kst(1), 1);
    wait_vmem_le<NJV / kWaves + NJK / kWaves>();
    // every wave's K(0) windows are in LDS; the barrier carries no release
    // fence (that would wait for V(0) and K(1) too), the acquire fence keeps
    // the LDS reads below it
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    f32x16_t sa[2], sb[2];
    if (nt_w > 0) {
#pragma unroll
        for (int i = 0; i < NS; ++i)
            sa[i & 1] = mfma32(k_operand(0, i), qf[i >> 1], i < 2 ? f32x16_t{} : sa[i & 1]);
        if (need_mask(0)) apply_mask(0, sa);
        float m4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) m4[k] = max8(sa, k);
        decide(rowmax(m4));
    }
    wait_vmem_all();
    __syncthreads();

    // iteration t: K(t+2) and V(t+1) are loaded into the stages K(t) and
    // V(t-1) left; S(t+1) is computed from K(t+1) beside the exponentials of
    // tile t, then O += P(t) V(t) beside the rest of them and the row max of
    // tile t+1.  One barrier per iteration.  A wave's last tile (LAST) has no
    // S(t+1) to compute, and when keys 32..63 of it are all past the wave's
    // visible keys (the causal diagonal, a key length) their exponentials and
    // P.V products are skipped too: those weights are exactly 0, so the result
    // is the same to the bit.
    auto refill = [&](int par, int t) {   // K(t+2), V(t+1); they land before the barrier
        dma_k(kst(par), t + 2);
        dma_v(vst(par ^ 1), t + 1);
    };
    auto step = [&](auto par_c, auto last_c, int t, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
        constexpr int par = decltype(par_c)::value;
        constexpr bool LAST = decltype(last_c)::value;
        refill(par, t);
        uint32_t pk[4][4];
        // row-sum partials of the pairs being made: those beside the S MFMAs,
        // then (folded into ts first) those beside the P.V MFMAs
        float rs[4] = {-0.f, -0.f, -0.f, -0.f};
        // last tile: keys 32..63 of it all past the wave's visible keys?
        bool half = false;
        if constexpr (LAST) {
            const int j0 = (tbase + t) * kBc;
            const int vis_last = CAUSAL ? min(kv_lim - 1, wq_last + off) : kv_lim - 1;
            half = j0 + 32 > vis_last;
        }
        // Guard rule, slow path for pairs [q0, q1) (whole chunks of 4 pairs):
        // the max of their scores, the reference moved to it where it grew
        // (o and l, which hold everything before these pairs, rescaled), the
        // pairs made again into r.  A reference that covers the pairs being
        // made is all the recurrence needs: pairs made later are checked
        // again.  Returns the rescale factor.
        [[maybe_unused]] auto redo = [&](auto q0_c, auto q1_c, float (&r)[4]) {
            constexpr int q0 = decltype(q0_c)::value, q1 = decltype(q1_c)::value;
            float mx = neg_inf();
#pragma unroll
            for (int k = q0 / 4; k < q1 / 4; ++k) mx = fmaxf(mx, max8(sc, k));
            const float alpha = decide(max_xor32(mx) * c);
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = -0.f;
#pragma unroll
            for (int q = q0; q < q1; ++q)
                if (!LAST || !half || q < 8) p_pair(sc, q, pk, r);
            return alpha;
        };
        u32x4_t kop[PD];
        if constexpr (!LAST) {
#pragma unroll
            for (int i = 0; i < PD; ++i) kop[i] = k_operand(par ^ 1, i);
        }
        if constexpr (kPrioPhase == 1) __builtin_amdgcn_s_setprio(1);
        if constexpr (kStagedPairs) {
            // pairs 0 .. NS-1 through the three-stage pipeline, two slots of
            // drain after the last MFMA
            float xa[3][2];
#pragma unroll
            for (int i = 0; i < NS + 2; ++i) {
                if constexpr (!LAST) {
                    if (i < NS) {
                        sn[i & 1] = mfma32(kop[i % PD], qf[i >> 1], i < 2 ? f32x16_t{} : sn[i & 1]);
                        if (i + PD < NS) kop[i % PD] = k_operand(par ^ 1, i + PD);
                    }
                }
                if (i < NS && (!LAST || !half || i < 8)) pair_args(sc, i, xa[i % 3]);
                if (i >= 1 && i - 1 < NS && (!LAST || !half || i - 1 < 8)) pair_exp(xa[(i - 1) % 3]);
                if (i >= 2 && (!LAST || !half || i - 2 < 8)) pair_keep(i - 2, xa[(i - 2) % 3], pk, rs);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                if constexpr (!LAST) {
                    sn[i & 1] = mfma32(kop[i % PD], qf[i >> 1], i < 2 ? f32x16_t{} : sn[i & 1]);
                    if (i + PD < NS) kop[i % PD] = k_operand(par ^ 1, i + PD);
                }
                if (!LAST || !half || i < 8) p_pair(sc, i, pk, rs);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (kPrioPhase == 1) __builtin_amdgcn_s_setprio(0);
        if constexpr (!LAST)
            if (need_mask(t + 1)) apply_mask(t + 1, sn);
        // Guard rule: the weights made so far (pairs 0 .. NS-1) are kept unless
        // some lane's sum of them reached the limit or a lane has no reference
        // yet; the pairs made beside the P.V MFMAs are checked the same way
        // before the MFMAs that use them.
        float ts = (rs[0] + rs[1]) + (rs[2] + rs[3]);
        if constexpr (GUARD) {
            if (!all_ref || __any(!(ts < kGuardLimit))) {
                redo(IntC<0>{}, IntC<NS>{}, rs);
                ts = (rs[0] + rs[1]) + (rs[2] + rs[3]);
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) rs[k] = -0.f;
        [[maybe_unused]] float m4[4];
        u32x4_t vop[PD];
#pragma unroll
        for (int i = 0; i < PD; ++i) vop[i] = v_operand(par, i);
        if constexpr (kPrioPhase == 2) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NP2; ++i) {
            const int ci = i / CB;
            if constexpr (GUARD && PAIRS2 > 0) {
                if (i == NP2 / 2 && (!LAST || !half)) {
                    const float ts2 = (rs[0] + rs[1]) + (rs[2] + rs[3]);
                    if (__any(!(ts2 < kGuardLimit)))
                        ts *= redo(IntC<NS>{}, IntC<16>{}, rs);   // the first pairs are in o already
                }
            }
            if (!LAST || !half || ci < 2)
                acc[i % CB] = mfma32(vop[i % PD], u32x4_t{pk[ci][0], pk[ci][1], pk[ci][2], pk[ci][3]},
                                     acc[i % CB]);
            if (i + PD < NP2) vop[i % PD] = v_operand(par, i + PD);
            if (i < PAIRS2 / 2 && (!LAST || !half)) {
                p_pair(sc, NS + 2 * i, pk, rs);
                p_pair(sc, NS + 2 * i + 1, pk, rs);
            }
            if constexpr (!LAST && !GUARD) {
                if (i >= NP2 - 4) {
                    m4[i - (NP2 - 4)] = max8(sn, i - (NP2 - 4));
                    pin(m4[i - (NP2 - 4)]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kPrioPhase == 2) __builtin_amdgcn_s_setprio(0);
        l += ts + ((rs[0] + rs[1]) + (rs[2] + rs[3]));
        if constexpr (!GUARD && !LAST) decide(rowmax(m4));
        wait_vmem_all();
        __syncthreads();
    };
    // every wave passes nloop barriers: nt_w in its own tiles (the last one by
    // the LAST step), the rest in the refill-only loop
    int t = 0;
    for (; t + 2 < nt_w; t += 2) {
        step(IntC<0>{}, BoolC<false>{}, t, sa, sb);
        step(IntC<1>{}, BoolC<false>{}, t + 1, sb, sa);
    }
    if (t + 2 == nt_w) {
        step(IntC<0>{}, BoolC<false>{}, t, sa, sb);
        step(IntC<1>{}, BoolC<true>{}, t + 1, sb, sa);
        t += 2;
    } else if (t + 1 == nt_w) {
        step(IntC<0>{}, BoolC<true>{}, t, sa, sb);
        ++t;
    }
    for (; t < nloop; ++t) {
        refill(t & 1, t);
        wait_vmem_all();
        __syncthreads();
    }
    if constexpr (KSPLIT > 1) {
        // groups 1.. hand their (reference, l, o) to group 0 through the V
        // stages (every wave is past its last LDS read and no load is in
        // flight): one 256-byte row per register, lane-indexed
        constexpr int RW = 16 * CB + 2;                      // rows per wave
        constexpr int R0 = (int)(sizeof(Vs0) / 256);         // rows in Vs0
        static_assert((KSPLIT - 1) * kWaves * RW <= 2 * R0, "merge rows do not fit the V stages");
        auto mrow = [&](int from, int k) -> float * {
            const int r = ((from - 1) * kWaves + wave) * RW + k;
            return (r < R0 ? (float *)Vs0 + 64 * r : (float *)Vs1 + 64 * (r - R0)) + lane;
        };
        if (grp > 0) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int v = 0; v < 16; ++v) *mrow(grp, 16 * cb + v) = acc[cb][v];
            *mrow(grp, 16 * CB) = ms;
            *mrow(grp, 16 * CB + 1) = l;
        }
        __syncthreads();
        if (grp > 0) return;
        // merge in group order ('Online Softmax & FlashAttention', Step 1):
        // common reference m = max(m0, m1), each side scaled by 2^(m_g - m),
        // 0 for a side without keys
#pragma unroll
        for (int from = 1; from < KSPLIT; ++from) {
            const float ms1 = *mrow(from, 16 * CB), l1 = *mrow(from, 16 * CB + 1);
            const float mm = fmaxf(ms, ms1);
            const float a0 = ms == neg_inf() ? 0.f : exp2_hw(ms - mm);
            const float a1 = ms1 == neg_inf() ? 0.f : exp2_hw(ms1 - mm);
            l = a0 * l + a1 * l1;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[cb][v] = a0 * acc[cb][v] + a1 * *mrow(from, 16 * cb + v);
            ms = mm;
        }
    }

    // epilogue: O = o / l (0 for a row without keys), LSE = ms + log2 l in nats (-inf then)
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
        if (g == 0) LSE[(size_t)bh * N + qrow] = lt > 0.f ? (ms + log2_hw(lt)) * kLn2 : neg_inf();
    }
}


template <int D, bool CAUSAL, int KSPLIT, int RULE>
hipError_t launch_one(const FwdArgs &a, int n_qtiles, long long nblocks, int order,
                      hipStream_t stream) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, KSPLIT, RULE>), dim3((unsigned)nblocks),
                       dim3(kThreads * KSPLIT), 0, stream, (const uint16_t *)a.Q,
                       (const uint16_t *)a.K, (const uint16_t *)a.V, (uint16_t *)a.O, a.LSE,
                       a.key_lens, a.H, a.N, a.Nk, n_qtiles, order, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_d(const FwdArgs &a, hipStream_t stream) {
    const int n_qtiles = (a.N + kBr - 1) / kBr;
    const long long BH = (long long)a.B * a.H;
    const long long nblocks = BH * n_qtiles;
    const int order = launch_order(a.B, a.H, CAUSAL, a.key_lens, 2ll * a.Nk * D * 2);
    // a grid of at most one block per CU leaves each CU with one four-wave
    // workgroup (one wave per SIMD): split every block's keys over two groups
    // of four waves instead.  Such a workgroup needs the LDS of two and runs
    // one per CU, so with more blocks than CUs it would take more dispatch
    // rounds than the unsplit grid (measured slower at 512 blocks).
    // rescale rules other than the default exist for the ablation only and
    // always run unsplit
    const int rule = rescale_rule();
    if (rule == kRuleEager) return launch_one<D, CAUSAL, 1, kRuleEager>(a, n_qtiles, nblocks, order, stream);
    if (rule == kRuleTau) return launch_one<D, CAUSAL, 1, kRuleTau>(a, n_qtiles, nblocks, order, stream);
    if (nblocks <= device_cu_count())
        return launch_one<D, CAUSAL, 2, kRuleGuard>(a, n_qtiles, nblocks, order, stream);
    return launch_one<D, CAUSAL, 1, kRuleGuard>(a, n_qtiles, nblocks, order, stream);
}

}  // namespace

namespace {
std::atomic<int> g_rescale_rule{kRuleGuard};
}  // namespace
void set_rescale_rule(int rule) {
    g_rescale_rule.store(rule == kRuleEager || rule == kRuleTau ? rule : kRuleGuard);
}
int rescale_rule() { return g_rescale_rule.load(std::memory_order_relaxed); }

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream) {
    if (a.d == 64) return a.causal ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
    return a.causal ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
}

}  // namespace fa
