// Stable LSD radix sort passes over uint32 keys with int32 values (internal
// to libspc; used for the kernel maps' processing orders and the point
// voxeliser's per-voxel point order).  One pass = k_rs_hist then
// k_rs_scatter on RS_BITS bits at `shift`; the host chains the passes over
// two ping-pong buffers.  A launch can carry the same pass of two
// independent sorts (RsPass): its first job[0].nb blocks serve job 0, the
// rest job 1, which halves the launches of a strided kernel map's two orders.
// Row counts are host values or, with rows < 0, a device count read at
// n_dev (treated as 0 when above cap).
#pragma once

#include "common.h"

namespace spc {
namespace {

constexpr int RS_THREADS = 512;              // threads per radix block (one per digit in the spine)
constexpr int RS_ITEMS = 4;                  // keys per thread in the radix passes
constexpr int RS_TILE = RS_THREADS * RS_ITEMS;  // keys per radix block
constexpr int RS_GROUP = 16;                 // radix blocks per group of the two-level offset sums
constexpr int RS_SPINE_GROUPS = 64;          // above this many groups a pass scans them once (k_rs_spine)
constexpr int RS_MAX_PASSES = 4;             // K <= 32 bits of mask, 9 bits per pass
constexpr int RS_BITS = 9;                   // digit width of the radix passes
constexpr int RS_BINS = 1 << RS_BITS;

__device__ __forceinline__ int32_t count_within(const uint32_t* n_dev, int64_t cap) {
    const uint32_t m = *n_dev;
    return int64_t(m) <= cap ? int32_t(m) : 0;
}

// One sort's arguments for one pass.
struct RsJob {
    const uint32_t* keys_in;
    const int32_t* vals_in;     // NULL: the identity (the row index)
    uint32_t* keys_out;
    int32_t* vals_out;
    int32_t* hist;              // [RS_BINS][nb] block counts
    int32_t* gsum;              // [RS_BINS][ng] group sums, zeroed beforehand
    int32_t* gtot;              // [RS_BINS] digit totals from k_rs_spine, or NULL (no spine)
    const uint32_t* n_dev;      // device row count when rows < 0
    int64_t cap;
    int32_t rows;
    int32_t nb, ng;             // radix blocks and block groups of this sort
};

// One pass of up to two sorts (job[1].nb == 0: one sort).
struct RsPass {
    RsJob job[2];
    int32_t shift;
};

// Lanes of this wave whose (valid) digit equals this lane's, from RS_BITS ballots.
__device__ __forceinline__ uint64_t digit_peers(bool valid, uint32_t d) {
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < RS_BITS; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bb = __ballot(valid && bit);
        peers &= bit ? bb : ~bb;
    }
    return peers;
}

// Radix sort.  A block owns RS_TILE consecutive keys; wave w of the block
// owns the contiguous run [w * RS_TILE / NW, (w + 1) * RS_TILE / NW), taken
// 64 at a time, so the block's keys are visited in index order per wave.
constexpr int RS_WAVES = RS_THREADS / WAVE;
constexpr int RS_PER_WAVE = RS_TILE / RS_WAVES;
static_assert(RS_THREADS == RS_BINS, "one thread per digit");

// Pass histogram.  Every block counts the digits (key >> shift) &
// (RS_BINS-1) of its tile into hist[d*nb + block] and adds them to the sums
// of its group of RS_GROUP blocks, gsum[d*ng + block/RS_GROUP] (zeroed
// beforehand).  rows < 0: the count at n_dev (0 when above cap).
__global__ __launch_bounds__(RS_THREADS) void k_rs_hist(RsPass P) {
    __shared__ int32_t h[RS_BINS];
    const bool second = int(blockIdx.x) >= P.job[0].nb;
    const RsJob& J = second ? P.job[1] : P.job[0];
    const int me = int(blockIdx.x) - (second ? P.job[0].nb : 0);
    const uint32_t* __restrict__ keys = J.keys_in;
    const int shift = P.shift;
    int32_t rows = J.rows;
    if (rows < 0) rows = count_within(J.n_dev, J.cap);
    const int32_t tile0 = int32_t(me) * RS_TILE;
    if (tile0 >= rows) return;  // uniform per block; later blocks are never read
    const int t = threadIdx.x;
    uint32_t k[RS_ITEMS];
#pragma unroll
    for (int r = 0; r < RS_ITEMS; ++r) k[r] = ld_clamped(keys, tile0 + r * RS_THREADS + t, rows);
    h[t] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RS_ITEMS; ++r)
        if (tile0 + r * RS_THREADS + t < rows) atomicAdd(h + ((k[r] >> shift) & (RS_BINS - 1)), 1);
    __syncthreads();
    const int c = h[t];
    J.hist[int64_t(t) * J.nb + me] = c;
    if (c) atomicAdd(J.gsum + int64_t(t) * J.ng + me / RS_GROUP, c);
}

// Rows a job sorts, and its groups that hold rows (later groups' sums stay 0).
__device__ __forceinline__ int32_t job_rows(const RsJob& J) {
    return J.rows < 0 ? count_within(J.n_dev, J.cap) : J.rows;
}
__device__ __forceinline__ int live_groups(const RsJob& J, int32_t rows) {
    return min(J.ng, int((int64_t(rows) + int64_t(RS_TILE) * RS_GROUP - 1) / (int64_t(RS_TILE) * RS_GROUP)));
}

// Pass spine, for sorts of many groups (J.gtot set): each digit's group sums
// become exclusive prefixes in place and the digit's total goes to gtot, so a
// scatter block reads one prefix and one total instead of every group's sum
// (a cost that grew with the square of the rows).  One wave per digit, four
// digits per block, RS_BINS / 4 blocks per job.
__global__ __launch_bounds__(256) void k_rs_spine(RsPass P) {
    constexpr int PER_JOB = RS_BINS / 4;
    const RsJob& J = int(blockIdx.x) >= PER_JOB ? P.job[1] : P.job[0];
    if (!J.gtot) return;  // uniform per block
    const int d = (int(blockIdx.x) % PER_JOB) * 4 + int(threadIdx.x) / WAVE;
    const int lane = threadIdx.x & (WAVE - 1);
    const int ng_live = live_groups(J, job_rows(J));
    int32_t* gs = J.gsum + int64_t(d) * J.ng;
    int carry = 0;
    for (int q0 = 0; q0 < ng_live; q0 += WAVE) {
        const int q = q0 + lane;
        const int v = q < ng_live ? gs[q] : 0;
        int x = v;  // inclusive scan over the wave
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (q < ng_live) gs[q] = carry + x - v;
        carry += __shfl(x, WAVE - 1);
    }
    if (lane == 0) J.gtot[d] = carry;
}

// Pass scatter, stable.  Slot base of digit d for this block: keys of
// smaller digits, plus digit-d keys of earlier groups (group sums) and of
// earlier blocks of this group (histogram columns); each wave adds the
// counts of earlier waves of the block, then ranks its keys among equal
// digits with RS_BITS ballots (computed once, for counting and writing) and
// writes them in order.  vals_in == NULL means the identity (row index).
__global__ __launch_bounds__(RS_THREADS) void k_rs_scatter(RsPass P) {
    __shared__ int32_t base[RS_WAVES][RS_BINS];
    __shared__ uint32_t skey[RS_TILE];
    __shared__ int32_t sval[RS_TILE];
    const bool second = int(blockIdx.x) >= P.job[0].nb;
    const RsJob& J = second ? P.job[1] : P.job[0];
    const int me = int(blockIdx.x) - (second ? P.job[0].nb : 0);
    const uint32_t* __restrict__ keys_in = J.keys_in;
    const int32_t* __restrict__ vals_in = J.vals_in;
    const int32_t* __restrict__ hist = J.hist;
    const int32_t* __restrict__ gsum = J.gsum;
    uint32_t* __restrict__ keys_out = J.keys_out;
    int32_t* __restrict__ vals_out = J.vals_out;
    const int shift = P.shift, ng = J.ng, nb = J.nb;
    int32_t rows = J.rows;
    if (rows < 0) rows = count_within(J.n_dev, J.cap);
    const int32_t tile0 = int32_t(me) * RS_TILE;
    if (tile0 >= rows) return;  // uniform per block
    const int t = threadIdx.x, lane = t & (WAVE - 1), wave = t / WAVE;
    // 0. the block's keys and values (coalesced, unconditional loads) and this
    //    thread's digit counts are all requested before any of them is used
    uint32_t kr[RS_ITEMS];
    int32_t vr[RS_ITEMS];
#pragma unroll
    for (int r = 0; r < RS_ITEMS; ++r) kr[r] = ld_clamped(keys_in, tile0 + r * RS_THREADS + t, rows);
    if (vals_in) {
#pragma unroll
        for (int r = 0; r < RS_ITEMS; ++r) vr[r] = ld_clamped(vals_in, tile0 + r * RS_THREADS + t, rows);
    } else {
#pragma unroll
        for (int r = 0; r < RS_ITEMS; ++r) vr[r] = tile0 + r * RS_THREADS + t;
    }
    // digit t: totals over the groups and the part before this block.  Only
    // the groups that hold rows have sums (blocks past the rows add nothing
    // to their zeroed sums), so a sort sized by a capacity far above its
    // rows reads just those
    const int g_me = me / RS_GROUP, b0 = g_me * RS_GROUP;
    const int ng_live = live_groups(J, rows);
    int tot = 0, before = 0;
    {
        const int32_t* gs = gsum + int64_t(t) * ng;
        const int32_t* hc = hist + int64_t(t) * nb;
        int hv[RS_GROUP];
#pragma unroll
        for (int u = 0; u < RS_GROUP; ++u) hv[u] = ld_clamped(hc, b0 + u, int64_t(me) + 1);
        if (J.gtot) {  // the spine's prefixes (uniform per block)
            tot = J.gtot[t];
            before = gs[g_me];
        }
        for (int q0 = 0; !J.gtot && q0 < ng_live; q0 += RS_GROUP) {
            int v[RS_GROUP];
#pragma unroll
            for (int u = 0; u < RS_GROUP; ++u) v[u] = ld_clamped(gs, q0 + u, ng_live);
#pragma unroll
            for (int u = 0; u < RS_GROUP; ++u) {
                tot += q0 + u < ng_live ? v[u] : 0;
                before += q0 + u < g_me ? v[u] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < RS_GROUP; ++u) before += b0 + u < me ? hv[u] : 0;
    }
#pragma unroll
    for (int r = 0; r < RS_ITEMS; ++r) {
        skey[r * RS_THREADS + t] = kr[r];
        sval[r * RS_THREADS + t] = vr[r];
    }
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) base[w][t] = 0;
    __shared__ int waves[RS_WAVES];
    int total;
    const int32_t my_off = block_exclusive_scan<RS_THREADS>(tot, waves, total) + before;
    // (the scan's barriers also publish the LDS keys and the cleared bases)
    // 1. per-wave digit counts; wave w owns keys [w*RS_PER_WAVE, (w+1)*RS_PER_WAVE) of the block
    const uint64_t lt = (1ull << lane) - 1ull;
    uint64_t peers[RS_ITEMS];
    uint32_t dig[RS_ITEMS];
#pragma unroll
    for (int r = 0; r < RS_ITEMS; ++r) {
        const int j = wave * RS_PER_WAVE + r * WAVE + lane;
        const bool valid = tile0 + j < rows;
        dig[r] = (skey[j] >> shift) & (RS_BINS - 1);
        peers[r] = digit_peers(valid, dig[r]);
        if (valid && (peers[r] & lt) == 0) base[wave][dig[r]] += int(__popcll(peers[r]));  // one leader per digit
    }
    __syncthreads();
    // 2. wave bases: block base + earlier waves of this block
    int run = my_off;
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) {
        const int c = base[w][t];
        base[w][t] = run;
        run += c;
    }
    __syncthreads();
    // 3. each wave writes its keys in order
#pragma unroll
    for (int r = 0; r < RS_ITEMS; ++r) {
        const int j = wave * RS_PER_WAVE + r * WAVE + lane;
        if (tile0 + j < rows) {
            const int rank = __popcll(peers[r] & lt);
            const int pos = base[wave][dig[r]] + rank;
            keys_out[pos] = skey[j];
            vals_out[pos] = sval[j];
            if (rank == 0) base[wave][dig[r]] += __popcll(peers[r]);
        }
    }
}

}  // namespace
}  // namespace spc
