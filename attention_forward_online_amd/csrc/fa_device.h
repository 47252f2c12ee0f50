// fa_device.h -- device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).
// exp(x) is evaluated as 2^(x * log2 e); the log2(e) factor is folded into
// the score scale once per launch.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// Two floats to two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed lo|hi.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Raw buffer resource over [base, base + bytes): a load at a byte offset
// >= bytes returns zeros (hardware range check), so ragged tiles need no
// branches.  0x00020000 is the gfx9-family descriptor word 3 (32-bit data).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ float buffer_load_f32(rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// The share of a ROWS x DMAX fp32 tile (rows of `d` valid floats, zero-filled
// to DMAX) that thread `tid` of a THREADS-thread workgroup copies from global
// memory to LDS: elements tid + THREADS p.  load() only issues the loads, so a
// caller can overlap them with work on the previous tile; a column at or past
// d, or a row past the buffer's range, reads 0 (hardware range check).
template <int ROWS, int DMAX, int THREADS>
struct F32TileStage {
    static constexpr int PER = ROWS * DMAX / THREADS;
    static_assert(ROWS * DMAX % THREADS == 0, "tile/thread mismatch");
    float v[PER];
    __device__ __forceinline__ void load(rsrc_t src, int row0, int d, int tid) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + THREADS * p, row = e / DMAX, col = e % DMAX;
            // a column at or past d gets an offset past any range (no branch)
            const uint32_t off = (uint32_t)((row0 + row) * d + col) * 4u | (col < d ? 0u : 0xfffffff0u);
            v[p] = buffer_load_f32(src, off);
        }
    }
    __device__ __forceinline__ void store(float *lds, int tid) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) lds[tid + THREADS * p] = v[p];
    }
};

// 16-byte buffer load straight into LDS (no register stage): lane l of the
// wave writes bytes lds + 16 l .. lds + 16 l + 15; a lane whose offset fails the
// range check writes zeros, an inactive lane writes nothing.  `lds` is
// wave-uniform (it goes to M0).  The write is tracked by the vector-memory
// counter: wait_vmem_all() and a barrier before other waves read it.
__device__ __forceinline__ void buffer_load_lds16(rsrc_t r, void *lds, uint32_t byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             byte_off, 0, 0, 0);
}

// Keep a value computed at this point of the instruction stream: an empty
// volatile asm reads and redefines the register, so the computation cannot
// be sunk past it towards its first use (used to interleave VALU work with
// matrix instructions that the scheduler would otherwise separate).
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane s supplies the LDS address of 4 consecutive 16-bit elements (a row
// chunk); lane L receives element L % 4 of the chunks of lanes L/4 + 4t,
// t = 0..3, as its element t.  A 4 x 16 block whose row r, column chunk q is
// read by lane 4r + q therefore arrives transposed: lane 4q + u holds column
// 4q + u of rows 0..3.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
__device__ __forceinline__ u32x2_t lds_read_tr16(const __attribute__((address_space(3))) uint16_t *p) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p));
}

// Wait until every vector-memory load of this wave has returned
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N vector-memory loads of this wave are outstanding (they
// complete in issue order for this count): s_waitcnt vmcnt(N), vmcnt split
// over bits 3:0 and 15:14.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// max(v, value of lane ^ 32) on the VALU (v_permlane32_swap exchanges the
// two 32-lane halves), without going through the LDS queue.
__device__ __forceinline__ float max_xor32(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// Value of lane (lane ^ mask) for masks < 64.
__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Value of lane (lane ^ M) for M = 1 or 2: a DPP quad permutation on the VALU
// (no LDS round trip, unlike a general shuffle).
template <int M>
__device__ __forceinline__ float quad_xor_f32(float v) {
    static_assert(M == 1 || M == 2, "quad exchange");
    constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
}

// Row order of a 32-row MFMA operand block: operand row r reads row perm32(r)
// (bits 2 and 3 swapped).  With it the 32x32 accumulator registers 8h..8h+7
// of lane half g hold rows 16h + 8g + 0..7 -- eight consecutive rows, which is
// the k-layout of the next MFMA's operand, so scores feed P.V (and P, dS feed
// the backward products) without any register shuffle.
__device__ __forceinline__ int perm32(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// D = A B + C on v_mfma_f32_32x32x16_bf16: A row / B column = lane % 32, the
// 8 k values of each lane at k offset 8 * (lane / 32); D column = lane % 32,
// rows 8(v/4) + 4(lane/32) + v%4 in register v.
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// The visible keys of batch b: its key length clamped to [0, Nk] (all Nk
// without key lengths).
__device__ __forceinline__ int visible_len(const int32_t *key_lens, int b, int Nk) {
    if (!key_lens) return Nk;
    int kl = key_lens[b];
    return kl < 0 ? 0 : (kl > Nk ? Nk : kl);
}

// Launch orders of a grid of BH heads x nblk blocks: workgroup id -> (head bh,
// rank of the block within its head).
//  kOrderPlain: rank-major, head-fastest.
//  kOrderXcd (BH a multiple of 8): head bh on XCD bh % 8 (the dispatcher deals
//    workgroup ids to the XCDs round-robin), so all blocks of a head share one
//    L2; within an XCD its heads go in groups of G (order >> 8, 0 = all of
//    them), rank-major within a group and one group after the other, so the
//    tiles the running blocks stream come from G heads at a time.
//  kOrderByKeyLen (per-batch key lengths, at most kMaxOrderBatches batches):
//    batch by batch, rank-major and head-fastest within a batch.  Up to 64
//    batches go in descending order of visible keys (ties by batch index): lane
//    i ranks batch i and the block's batch is the one whose rank is its
//    position.  More batches go with those that have keys first, each part in
//    index order, from one 64-bit mask of "has keys" per 64 batches (with no
//    batch empty, the head-per-XCD or plain order instead).  Why: each
//    XCD sends its even- and odd-numbered workgroups to different halves of its
//    CUs, so an order that alternates a batch without keys with one with keys
//    leaves half the CUs idle; this way the blocks with work go out first.
//    Every lane of the wave must be active.
constexpr int kOrderPlain = 0, kOrderXcd = 1, kOrderByKeyLen = 2;
constexpr int kMaxOrderBatches = 1024;     // batches the key-length order handles
__device__ __forceinline__ void block_in_order(int bid, int BH, int nblk, int order, int H,
                                               const int32_t *key_lens, int Nk, int &bh,
                                               int &rank) {
    if (order == kOrderByKeyLen) {
        const int lane = threadIdx.x & 63;
        const int nb = BH / H, per_b = H * nblk;
        const int pos = bid / per_b, rem = bid - pos * per_b;
        rank = rem / H;
        if (nb <= 64) {
            const int len = lane < nb ? visible_len(key_lens, lane, Nk) : -1;
            int my_rank = 0;
            for (int i = 0; i < nb; ++i) {
                const int other = __builtin_amdgcn_readlane(len, i);
                my_rank += (other > len || (other == len && i < lane)) ? 1 : 0;
            }
            const unsigned long long hit = __ballot(lane < nb && my_rank == pos);
            bh = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit)) * H + (rem - rank * H);
            return;
        }
        // more batches: one mask of "has keys" per 64 batches, all loads issued
        // together; with some batch empty, the pos-th batch of its part
        unsigned long long has[kMaxOrderBatches / 64];
        int with = 0;
#pragma unroll
        for (int c = 0; c < kMaxOrderBatches / 64; ++c) {
            const int i = 64 * c + lane;
            has[c] = __ballot(i < nb && visible_len(key_lens, i, Nk) > 0);
            with += __builtin_popcountll(has[c]);
        }
        if (with < nb) {
            const bool want = pos < with;
            int left = want ? pos : pos - with;   // batches of the part still to pass
            int batch = 0;
#pragma unroll
            for (int c = 0; c < kMaxOrderBatches / 64; ++c) {
                const int cnt = min(64, max(nb - 64 * c, 0));
                const unsigned long long valid = cnt == 64 ? ~0ull : ((1ull << cnt) - 1ull);
                const unsigned long long m = want ? has[c] : (~has[c] & valid);
                const int n = __builtin_popcountll(m);
                if (left >= 0 && left < n) {
                    // the left-th set bit of m: the lane with that many set bits below it
                    const unsigned long long below = m & ((1ull << lane) - 1ull);
                    const unsigned long long hit =
                        __ballot(((m >> lane) & 1ull) && __builtin_popcountll(below) == left);
                    batch = 64 * c + __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
                }
                left -= n;
            }
            bh = batch * H + (rem - rank * H);
            return;
        }
        // every batch has keys: nothing to move, the order below applies
        order = BH % 8 == 0 ? kOrderXcd : kOrderPlain;
    }
    if ((order & 0xff) == kOrderXcd) {
        const int hpx = BH >> 3, slot = bid >> 3;
        const int G = (order >> 8) > 0 ? (order >> 8) : hpx;   // hpx is a multiple of G
        const int grp = slot / (G * nblk), r = slot - grp * (G * nblk);
        rank = r / G;
        bh = (grp * G + r % G) * 8 + (bid & 7);
    } else {
        rank = bid / BH;
        bh = bid % BH;
    }
}

// The launch order for a grid: by key length for non-causal grids with key
// lengths, else head-per-XCD when B*H is a multiple of 8.  Causal grids keep
// their own longest-first order within each head.  stream_bytes: the bytes
// each block of a head streams from the head's shared tensors (K and V for
// the forward).  When an XCD's heads together stream more than its L2 holds
// (4 MiB), they go in groups that fit (at least one head): rank-major over
// all of them would keep re-reading tiles that other heads evicted (measured
// on B1 H32 N=Nk=8192 d=128 causal: 384 -> 211 MB read per call, time
// unchanged; heads that fit keep the rank-major order, which balances the
// causal tail better).
constexpr long long kXcdL2Bytes = 4ll << 20;
__host__ inline int launch_order(long long B, long long H, bool causal, const int32_t *key_lens,
                                 long long stream_bytes) {
    if (key_lens && !causal && B <= kMaxOrderBatches) return kOrderByKeyLen;
    if ((B * H) % 8 != 0) return kOrderPlain;
    const long long hpx = B * H / 8;
    long long g = stream_bytes > 0 ? kXcdL2Bytes / stream_bytes : hpx;
    if (g >= hpx) return kOrderXcd;
    if (g < 1) g = 1;
    while (hpx % g) --g;
    return kOrderXcd | (int)(g << 8);
}

}  // namespace fa
