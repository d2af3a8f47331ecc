// Kernel-map construction on the GPU: hash build, per-offset probes, strided
// output sites, CSR pair lists and mask-sorted processing orders.
//
// Hash table: open addressing with linear probing over 64-bit slots that pack
// (key << 32) | row, so one 8-byte load answers a probe and one 64-bit CAS
// claims a slot (the single-slot table of spconv's hash.HashTable on the
// context7 spconv page).  Keys are ((b*Z + z)*Y + y)*X + x, the packing of the
// MLX sparse/conv.py page's build_indice_map, bounded below 2^32 so the
// all-ones slot can mark "empty".  Capacity is a power of two >= 4N.
//
// Strided output sites are marked in a bitmap over the output grid; a
// per-word exclusive prefix of popcounts then gives, for any output site, its
// row in (b, z, y, x) order (rank = prefix[word] + popcount of the lower bits),
// so sorted output coordinates need no sort and no second table.  The
// input-side map follows from the ranks, and the output-side map is its
// transpose, scattered from it (no hash probes at all on the strided path;
// the hash still detects duplicate inputs).
//
// Maps are row-major [rows][K].  A row pass builds each row's neighbour mask
// and the per-(offset, block) hit counts; pair lists are compacted in
// (offset, row) order by one exclusive scan and an ordered ballot/prefix write
// pass.  The processing order is a stable LSD radix sort of (mask, row) with
// 9-bit digits: per pass a block histogram whose last block scans the
// histogram matrix into slot offsets, and a stable scatter.
#include <stdio.h>

#include <algorithm>

#include "common.h"
#include "radix.h"

namespace spc {
namespace {

constexpr uint64_t EMPTY_SLOT = ~0ull;
constexpr int KB = 256;          // threads per block of the per-row / per-entry kernels
constexpr int WORDS_PER_THREAD = 8;
constexpr int SCAN_THREADS = 256;            // small blocks (16 KB of LDS) that fit beside convolution tiles
constexpr int SCAN_PER_THREAD = 16;
constexpr int MASK_BITS = 32;                // orders are built for K <= 32
constexpr int MAX_K = 343;                   // up to 7 x 7 x 7 offsets
constexpr uint64_t OCC_FILTER_CELLS_PER_ROW = 8192;        // hash filter: at most 1 KiB of bitmap per row
constexpr uint64_t OCC_FILTER_MAX_BYTES = uint64_t(1) << 30;
// strided output sites: a byte per site (plain stores) for output grids of at
// most this many sites per input row and this many sites in all; otherwise
// the bitmap directly (atomic ORs)
constexpr uint64_t BYTEMAP_SITES_PER_ROW = 32;
constexpr uint64_t BYTEMAP_MAX_SITES = uint64_t(1) << 29;

struct KGeom {
    int32_t batch, Z, Y, X;      // input grid
    int32_t kz, ky, kx;
    int32_t sz, sy, sx;
    int32_t pz, py, px;
    int32_t dz, dy, dx;
    int32_t oz, oy, ox;          // output grid (equal to the input grid for subm)
    // reciprocals for division by these invariants (qdiv; 0 for a divisor of 1):
    // K, the strides, and the output grid's x extent, plane and volume
    uint64_t mK, msz, msy, msx, mox, mplane, mvol;
    int32_t occ;                 // input occupancy bitmap in use (see make_plan)
    int32_t dense;               // the index grid is the table (with the bitmap); else the hash is
};

// ceil(2^64 / d) for d >= 2, 0 for d == 1 (see qdiv)
inline uint64_t recip64(uint64_t d) { return d <= 1 ? 0 : ~uint64_t(0) / d + 1; }

// floor(n / d) from m = recip64(d): n * m / 2^64 exceeds n / d by less than
// n / 2^64 < 2^-32 < 1 / d, which never carries past the next integer.
__device__ __forceinline__ uint32_t qdiv(uint32_t n, uint64_t m) {
    return m ? uint32_t(__umul64hi(uint64_t(n), m)) : n;
}

// Offsets k < K as packed (kz << 6 | ky << 3 | kx), z slowest, into LDS.
__device__ __forceinline__ void offset_table(uint32_t* ktab, const KGeom& g, int K) {
    for (int k = threadIdx.x; k < K; k += blockDim.x)
        ktab[k] = uint32_t((k / (g.kx * g.ky)) << 6 | ((k / g.kx) % g.ky) << 3 | (k % g.kx));
    __syncthreads();
}

// Header at the start of the workspace.
enum { H_FLAGS = 0, H_NOUT = 1, H_TOT = 32, H_WORDS = 64 };   // H_TOT: per-offset pair totals (K <= 32)

__device__ __forceinline__ uint32_t mix32(uint32_t k) {
    // murmur3's 32-bit finaliser
    k ^= k >> 16;
    k *= 0x85ebca6bu;
    k ^= k >> 13;
    k *= 0xc2b2ae35u;
    k ^= k >> 16;
    return k;
}

// Home slot of a key: the four keys of one block of x (key >> 2) hash together
// and take four adjacent slots (32 bytes, inside one cache line), so the
// probes of neighbours along x, made by consecutive threads, share lines.
__device__ __forceinline__ uint32_t home_slot(uint32_t key) { return (mix32(key >> 2) << 2) | (key & 3u); }

__device__ __forceinline__ bool in_grid(const int4 c, const KGeom& g) {
    return (unsigned)c.x < (unsigned)g.batch && (unsigned)c.y < (unsigned)g.Z &&
           (unsigned)c.z < (unsigned)g.Y && (unsigned)c.w < (unsigned)g.X;
}

__device__ __forceinline__ uint32_t in_key(int b, int z, int y, int x, const KGeom& g) {
    return uint32_t(((uint64_t(b) * g.Z + z) * g.Y + y) * g.X + x);
}

__device__ __forceinline__ uint32_t out_key(int b, int z, int y, int x, const KGeom& g) {
    return uint32_t(((uint64_t(b) * g.oz + z) * g.oy + y) * g.ox + x);
}

__device__ __forceinline__ void table_insert(uint64_t* table, uint32_t mask, uint32_t key,
                                             uint32_t row, uint32_t* flags) {
    const unsigned long long slot = (static_cast<unsigned long long>(key) << 32) | row;
    uint32_t h = home_slot(key) & mask;
    // at most N of the >= 4N slots are ever taken, so an empty slot is always found
    for (uint32_t step = 0; step <= mask; ++step) {
        unsigned long long prev =
            atomicCAS(reinterpret_cast<unsigned long long*>(table + h), EMPTY_SLOT, slot);
        if (prev == EMPTY_SLOT) return;
        if (uint32_t(prev >> 32) == key) {
            atomicOr(flags, SPC_COORD_DUPLICATE);
            return;
        }
        h = (h + 1) & mask;
    }
}

__device__ __forceinline__ int32_t table_find(const uint64_t* __restrict__ table, uint32_t mask,
                                              uint32_t key) {
    uint32_t h = home_slot(key) & mask;
    for (uint32_t step = 0; step <= mask; ++step) {
        const uint64_t v = table[h];
        if (v == EMPTY_SLOT) return -1;
        if (uint32_t(v >> 32) == key) return int32_t(uint32_t(v));
        h = (h + 1) & mask;
    }
    return -1;
}

// Output-row count M as the later kernels see it: 0 when it exceeds the
// caller's capacity (the host then reports SPC_ERR_CAPACITY).
__device__ __forceinline__ int32_t rows_within(const uint32_t* hdr, int64_t cap) {
    const uint32_t m = hdr[H_NOUT];
    return int64_t(m) <= cap ? int32_t(m) : 0;
}

// ---------------------------------------------------------------- kernels

// Fills `cap` hash slots with the empty marker; zeroes the output bitmap, the
// occupancy bitmap, the header, the caller's coordinate flags (NULL ok; later
// kernels OR their findings in) and `zero` (word counts multiples of 4).
__global__ void k_clear(uint64_t* __restrict__ table, int64_t cap, uint32_t* __restrict__ bitmap,
                        int64_t nwords, uint32_t* __restrict__ occ, int64_t occ_words, uint32_t* __restrict__ hdr,
                        int32_t* coord_err, int32_t* __restrict__ zero, int64_t nzero) {
    // (a strided map with a byte map passes the byte map here as the bitmap,
    // nwords counting its 4-byte words)
    const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    if (t < H_WORDS) hdr[t] = 0u;
    if (coord_err && t == 0) *coord_err = 0;
    u32x4 ones = {~0u, ~0u, ~0u, ~0u};
    for (int64_t i = t; i < cap / 2; i += stride) st16(table + 2 * i, ones);
    for (int64_t i = t; i < nwords / 4; i += stride) st16(bitmap + 4 * i, zero4());
    for (int64_t i = t; i < occ_words / 4; i += stride) st16(occ + 4 * i, zero4());
    for (int64_t i = t; i < nzero / 4; i += stride) st16(zero + 4 * i, zero4());
}

// Fills rows [0, M) of a [rows][K] map with -1 (M read on the device).
__global__ void k_fill_map(int32_t* __restrict__ map, int K, int64_t cap, const uint32_t* hdr) {
    const int64_t n = int64_t(rows_within(hdr, cap)) * K;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) map[i] = -1;
}

// Inserts every in-range input row; flags bad and duplicate rows.  For a
// strided geometry it also sets the bitmap bit of every output site the row
// reaches: o = (c + pad - k*dil) / stride per axis, exact and inside the grid.
template <bool STRIDED>
__global__ __launch_bounds__(KB) void k_insert(const int4* __restrict__ coords, int32_t n, KGeom g,
                                               uint64_t* table, uint32_t mask, uint32_t* occ,
                                               uint32_t* bitmap, uint8_t* sites, uint32_t* hdr) {
    const int32_t i = blockIdx.x * KB + threadIdx.x;
    if (i >= n) return;
    const int4 c = coords[i];
    if (!in_grid(c, g)) {
        atomicOr(hdr + H_FLAGS, SPC_COORD_OUT_OF_RANGE);
        return;
    }
    const uint32_t key = in_key(c.x, c.y, c.z, c.w, g);
    if (g.dense) {
        const uint32_t bit = 1u << (key & 31u);
        if (STRIDED) {  // a cell whose bit was already set is a duplicate (the host reads it with the count)
            if (atomicOr(occ + (key >> 5), bit) & bit) atomicOr(hdr + H_FLAGS, SPC_COORD_DUPLICATE);
        } else {        // no round trip: the SubM row kernel finds duplicates (its own cell holds another row)
            atomicOr(occ + (key >> 5), bit);
        }
        reinterpret_cast<int32_t*>(table)[key] = i;
    } else {
        // the hash flags duplicates itself; its bitmap filter only needs the bit
        if (g.occ) atomicOr(occ + (key >> 5), 1u << (key & 31u));
        table_insert(table, mask, key, uint32_t(i), hdr + H_FLAGS);
    }
    if (!STRIDED) return;
    int oz[8], oy[8], ox[8];
    int nz = 0, ny = 0, nx = 0;
    for (int k = 0; k < g.kz; ++k) {
        const int num = c.y + g.pz - k * g.dz;
        const int q = num >= 0 ? int(qdiv(uint32_t(num), g.msz)) : -1;
        if (q >= 0 && q * g.sz == num && q < g.oz && nz < 8) oz[nz++] = q;
    }
    for (int k = 0; k < g.ky; ++k) {
        const int num = c.z + g.py - k * g.dy;
        const int q = num >= 0 ? int(qdiv(uint32_t(num), g.msy)) : -1;
        if (q >= 0 && q * g.sy == num && q < g.oy && ny < 8) oy[ny++] = q;
    }
    for (int k = 0; k < g.kx; ++k) {
        const int num = c.w + g.px - k * g.dx;
        const int q = num >= 0 ? int(qdiv(uint32_t(num), g.msx)) : -1;
        if (q >= 0 && q * g.sx == num && q < g.ox && nx < 8) ox[nx++] = q;
    }
    if (sites) {  // a byte per site: plain stores, which concurrent rows may repeat
        for (int a = 0; a < nz; ++a)
            for (int b = 0; b < ny; ++b) {
                const uint32_t base = out_key(c.x, oz[a], oy[b], 0, g);
                for (int d = 0; d < nx; ++d) sites[base + uint32_t(ox[d])] = 1;
            }
        return;
    }
    // sites along x share a bitmap word mostly: one atomic per word touched
    for (int a = 0; a < nz; ++a)
        for (int b = 0; b < ny; ++b) {
            const uint32_t base = out_key(c.x, oz[a], oy[b], 0, g);
            uint32_t word = ~0u, bits = 0;
            for (int d = 0; d < nx; ++d) {
                const uint32_t key = base + uint32_t(ox[d]);
                if ((key >> 5) != word) {
                    if (bits) atomicOr(bitmap + word, bits);
                    word = key >> 5;
                    bits = 0;
                }
                bits |= 1u << (key & 31u);
            }
            if (bits) atomicOr(bitmap + word, bits);
        }
}

// Submanifold probes, one thread per map entry t = i*K + k: nbr[t] = row at
// coords[i] + d_k, else -1, with d_k = (kz - KZ/2, ky - KY/2, kx - KX/2), z
// slowest.  Consecutive threads write consecutive entries.
__global__ __launch_bounds__(KB) void k_subm_probe(const int4* __restrict__ coords, int32_t n, KGeom g,
                                                   const uint64_t* __restrict__ table, uint32_t mask,
                                                   const uint32_t* __restrict__ occ, int32_t* __restrict__ nbr,
                                                   const uint32_t* hdr, int32_t* coord_err) {
    __shared__ uint32_t ktab[MAX_K];
    const int K = g.kz * g.ky * g.kx;
    offset_table(ktab, g, K);
    const int64_t t = int64_t(blockIdx.x) * KB + threadIdx.x;
    if (coord_err && t == 0 && hdr[H_FLAGS]) atomicOr(coord_err, int32_t(hdr[H_FLAGS]));
    if (t >= int64_t(n) * K) return;
    const int32_t i = int32_t(qdiv(uint32_t(t), g.mK));  // K * n < 2^31
    const int k = int(t - int64_t(i) * K);
    const uint32_t kk = ktab[k];
    const int kx = kk & 7, ky = (kk >> 3) & 7, kz = kk >> 6;
    int32_t v = -1;
    const int4 c = coords[i];
    if (in_grid(c, g)) {
        const int z = c.y + kz - g.kz / 2, y = c.z + ky - g.ky / 2, x = c.w + kx - g.kx / 2;
        if (kz == g.kz / 2 && ky == g.ky / 2 && kx == g.kx / 2) {
            v = i;
            // the index grid's insert did not check: another row in this cell is a duplicate
            if (g.dense && reinterpret_cast<const int32_t*>(table)[in_key(c.x, c.y, c.z, c.w, g)] != i && coord_err)
                atomicOr(coord_err, SPC_COORD_DUPLICATE);
        } else if ((unsigned)z < (unsigned)g.Z && (unsigned)y < (unsigned)g.Y && (unsigned)x < (unsigned)g.X) {
            const uint32_t key = in_key(c.x, z, y, x, g);
            if (g.occ && !((occ[key >> 5] >> (key & 31u)) & 1u))
                v = -1;
            else if (!g.dense)
                v = table_find(table, mask, key);
            else
                v = reinterpret_cast<const int32_t*>(table)[key];
        }
    }
    nbr[t] = v;
}

// Popcount of each thread's WORDS_PER_THREAD bitmap words, summed per block
// into block_sums and added to *total (zeroed beforehand).
__global__ __launch_bounds__(KB) void k_bitmap_count(uint32_t* __restrict__ bitmap, int64_t nwords,
                                                     const uint8_t* __restrict__ sites,
                                                     int32_t* __restrict__ block_sums, uint32_t* total) {
    __shared__ int32_t red[KB / WAVE];
    const int64_t w0 = (int64_t(blockIdx.x) * KB + threadIdx.x) * WORDS_PER_THREAD;
    int s = 0;
    if (w0 < nwords) {
        u32x4 a, b;
        if (sites) {
            // the byte map (bytes 0 or 1) into the thread's bitmap words: 16
            // bytes give 16 bits, byte j bit j
            uint32_t w[WORDS_PER_THREAD];
            const uint8_t* src = sites + w0 * 32;
#pragma unroll
            for (int q = 0; q < WORDS_PER_THREAD; ++q) {
                const u32x4 lo = ld16(src + q * 32), hi = ld16(src + q * 32 + 16);
                const uint32_t v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                uint32_t bits = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    bits |= ((v[e] & 1u) | ((v[e] >> 7) & 2u) | ((v[e] >> 14) & 4u) | ((v[e] >> 21) & 8u)) << (4 * e);
                w[q] = bits;
            }
            a = u32x4{w[0], w[1], w[2], w[3]};
            b = u32x4{w[4], w[5], w[6], w[7]};
            st16(bitmap + w0, a);
            st16(bitmap + w0 + 4, b);
        } else {
            a = ld16(bitmap + w0);
            b = ld16(bitmap + w0 + 4);
        }
        s = __popc(a.x) + __popc(a.y) + __popc(a.z) + __popc(a.w) + __popc(b.x) + __popc(b.y) +
            __popc(b.z) + __popc(b.w);
    }
    for (int off = WAVE / 2; off > 0; off >>= 1) s += __shfl_down(s, off);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int w = 0; w < KB / WAVE; ++w) t += red[w];
        block_sums[blockIdx.x] = t;
        if (t) atomicAdd(total, uint32_t(t));
    }
}

// Exclusive scan of data[0, L) in place, in chunks of SCAN_THREADS *
// SCAN_PER_THREAD values staged through LDS (coalesced loads and stores;
// each thread scans a contiguous run of the chunk).  Workgroup b of a larger
// grid scans its own segment data[b*L, (b+1)*L) (the rows of a [K][nblk]
// count matrix, one per offset).  With ptr != NULL (one workgroup),
// ptr[k] = data[k * nblk] (after the scan) for k < K and ptr[K] = total: the
// CSR offsets of a (offset, block) count matrix.  With total_out != NULL the
// segment's total is stored at total_out[b].
__global__ __launch_bounds__(SCAN_THREADS) void k_scan(int32_t* __restrict__ data, int64_t L, int32_t* ptr,
                                                       int K, int64_t nblk, uint32_t* total_out) {
    constexpr int CH = SCAN_THREADS * SCAN_PER_THREAD;
    data += int64_t(blockIdx.x) * L;
    __shared__ int waves[SCAN_THREADS / WAVE];
    __shared__ int buf[CH];
    int carry = 0;
    for (int64_t base = 0; base < L; base += CH) {
        {
            int v[SCAN_PER_THREAD];
#pragma unroll
            for (int e = 0; e < SCAN_PER_THREAD; ++e) v[e] = ld_clamped(data, base + e * SCAN_THREADS + threadIdx.x, L);
#pragma unroll
            for (int e = 0; e < SCAN_PER_THREAD; ++e) {
                const int j = e * SCAN_THREADS + threadIdx.x;
                buf[j] = base + j < L ? v[e] : 0;
            }
        }
        __syncthreads();
        int v[SCAN_PER_THREAD];
        int s = 0;
#pragma unroll
        for (int e = 0; e < SCAN_PER_THREAD; ++e) {
            v[e] = buf[threadIdx.x * SCAN_PER_THREAD + e];
            s += v[e];
        }
        int tot;
        int run = carry + block_exclusive_scan<SCAN_THREADS>(s, waves, tot);
#pragma unroll
        for (int e = 0; e < SCAN_PER_THREAD; ++e) {
            buf[threadIdx.x * SCAN_PER_THREAD + e] = run;
            run += v[e];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < SCAN_PER_THREAD; ++e) {
            const int j = e * SCAN_THREADS + threadIdx.x;
            if (base + j < L) data[base + j] = buf[j];
        }
        carry += tot;
        __syncthreads();
    }
    if (ptr) {
        for (int k = threadIdx.x; k < K; k += SCAN_THREADS) ptr[k] = nblk > 0 ? data[int64_t(k) * nblk] : 0;
        if (threadIdx.x == 0) ptr[K] = carry;
    }
    if (total_out && threadIdx.x == 0) total_out[blockIdx.x] = uint32_t(carry);
}

// The output row count into the caller's device word, for the form of the
// call that does not wait: the strided count as the map kernels read it
// (hdr), or a known count (SubM: the input rows).
__global__ void k_publish_count(const uint32_t* hdr, int32_t known, int32_t* n_out_dev) {
    if (threadIdx.x == 0) n_out_dev[0] = hdr ? int32_t(hdr[H_NOUT]) : known;
}

// Writes each word's exclusive rank prefix and the output coordinates of
// its set bits, in (b, z, y, x) order (coordinates only if M <= cap).  The
// block's first rank is block_offs[block] when `scanned`, else the sum of
// the earlier blocks' counts in block_offs, added up here (few blocks).
__global__ __launch_bounds__(KB) void k_bitmap_emit(const uint32_t* __restrict__ bitmap, int64_t nwords,
                                                    const int32_t* __restrict__ block_offs, int32_t scanned,
                                                    uint32_t* __restrict__ prefix, int4* __restrict__ out_coords,
                                                    int64_t cap, const uint32_t* hdr, KGeom g) {
    __shared__ int waves[KB / WAVE];
    const int64_t w0 = (int64_t(blockIdx.x) * KB + threadIdx.x) * WORDS_PER_THREAD;
    uint32_t w[WORDS_PER_THREAD] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (w0 < nwords) {
        const u32x4 a = ld16(bitmap + w0), b = ld16(bitmap + w0 + 4);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
    int first;
    if (scanned) {
        first = block_offs[blockIdx.x];
    } else {
        int e = 0;
        for (int j = threadIdx.x; j < int(blockIdx.x); j += KB) e += block_offs[j];
        block_exclusive_scan<KB>(e, waves, first);
    }
    int s = 0;
    for (int j = 0; j < WORDS_PER_THREAD; ++j) s += __popc(w[j]);
    int total;
    int run = first + block_exclusive_scan<KB>(s, waves, total);
    if (w0 >= nwords) return;
    const bool emit = int64_t(hdr[H_NOUT]) <= cap;
    const uint32_t plane = uint32_t(g.oy) * uint32_t(g.ox), vol = plane * uint32_t(g.oz);
    for (int j = 0; j < WORDS_PER_THREAD; ++j) {
        prefix[w0 + j] = uint32_t(run);
        uint32_t bits = w[j];
        if (!emit || !bits) continue;
        // the word's first site, decoded once; its bits are consecutive x
        const uint32_t key0 = uint32_t(w0 + j) * 32u;
        const uint32_t b0 = qdiv(key0, g.mvol), r = key0 - b0 * vol;
        const uint32_t z0 = qdiv(r, g.mplane), r2 = r - z0 * plane;
        const uint32_t y0 = qdiv(r2, g.mox), x0 = r2 - y0 * uint32_t(g.ox);
        while (bits) {
            const uint32_t bit = __ffs(bits) - 1;
            bits &= bits - 1;
            uint32_t x = x0 + bit, y = y0, z = z0, b = b0;
            while (x >= uint32_t(g.ox)) {  // carry into y, z, b
                x -= uint32_t(g.ox);
                if (++y == uint32_t(g.oy)) {
                    y = 0;
                    if (++z == uint32_t(g.oz)) {
                        z = 0;
                        ++b;
                    }
                }
            }
            out_coords[run++] = make_int4(int(b), int(z), int(y), int(x));
        }
    }
}

// Strided maps, one thread per input-side entry t = i*K + k: the output site
// o = (c + pad - k*dil) / stride (exact, inside the grid) has row
// rank(o); nbr_in[t] = that row (or -1), and the output-side map gets the
// transposed entry nbr[row*K + k] = i (it was filled with -1 before).
__global__ __launch_bounds__(KB) void k_strided_maps(const int4* __restrict__ coords, int32_t n, int64_t cap,
                                                     KGeom g, const uint32_t* __restrict__ bitmap,
                                                     const uint32_t* __restrict__ prefix,
                                                     int32_t* __restrict__ nbr, int32_t* __restrict__ nbr_in,
                                                     const uint32_t* hdr, int32_t* coord_err) {
    __shared__ uint32_t ktab[MAX_K];
    const int K = g.kz * g.ky * g.kx;
    offset_table(ktab, g, K);
    const int64_t t = int64_t(blockIdx.x) * KB + threadIdx.x;
    if (coord_err && t == 0 && hdr[H_FLAGS]) atomicOr(coord_err, int32_t(hdr[H_FLAGS]));
    if (t >= int64_t(n) * K || int64_t(hdr[H_NOUT]) > cap) return;
    const int32_t i = int32_t(qdiv(uint32_t(t), g.mK));  // K * n < 2^31
    const int k = int(t - int64_t(i) * K);
    const uint32_t kk = ktab[k];
    const int kx = kk & 7, ky = (kk >> 3) & 7, kz = kk >> 6;
    const int4 c = coords[i];
    int32_t v = -1;
    const int nz = c.y + g.pz - kz * g.dz, ny = c.z + g.py - ky * g.dy, nx = c.w + g.px - kx * g.dx;
    const int oz = nz >= 0 ? int(qdiv(uint32_t(nz), g.msz)) : -1;
    const int oy = ny >= 0 ? int(qdiv(uint32_t(ny), g.msy)) : -1;
    const int ox = nx >= 0 ? int(qdiv(uint32_t(nx), g.msx)) : -1;
    if (in_grid(c, g) && oz >= 0 && oy >= 0 && ox >= 0 && oz * g.sz == nz && oy * g.sy == ny && ox * g.sx == nx) {
        if (oz < g.oz && oy < g.oy && ox < g.ox) {
            const uint32_t key = out_key(c.x, oz, oy, ox, g);
            const uint32_t word = key >> 5, bit = key & 31u;
            v = int32_t(prefix[word] + __popc(bitmap[word] & ((1u << bit) - 1u)));
            nbr[int64_t(v) * K + k] = i;
        }
    }
    if (nbr_in) nbr_in[t] = v;
}

// One thread per map row: the neighbour mask (bit k set iff entry k >= 0,
// for K <= 32) into keys[row], and per offset the block's hit count into
// counts[k*nblk + block] (wave counts summed with LDS atomics, one barrier).
// The block's rows are first copied to LDS with coalesced loads (for
// K <= ROWPASS_KMAX); a row stride of K words is conflict-free for odd K.
// rows < 0: read M from the header.
constexpr int ROWPASS_KMAX = 27;
constexpr int64_t EMIT_SUM_BLOCKS = 2048;   // up to this many bitmap blocks, emit sums the earlier counts itself

__global__ __launch_bounds__(KB) void k_row_pass(const int32_t* __restrict__ map, int32_t rows, int K,
                                                 int64_t cap, const uint32_t* hdr, uint32_t* __restrict__ keys,
                                                 int32_t* __restrict__ counts) {
    __shared__ int32_t stage[KB * ROWPASS_KMAX];
    __shared__ int32_t cnt[MAX_K];
    if (rows < 0) rows = rows_within(hdr, cap);
    const int32_t row0 = blockIdx.x * KB;
    const int32_t r = row0 + threadIdx.x;
    const bool live = r < rows;
    const bool staged = K <= ROWPASS_KMAX;
    for (int k = threadIdx.x; k < K; k += KB) cnt[k] = 0;
    if (staged && row0 < rows) {
        const int64_t lo = int64_t(row0) * K, hi = int64_t(min(rows, row0 + KB)) * K;
        int32_t v[ROWPASS_KMAX];
#pragma unroll
        for (int e = 0; e < ROWPASS_KMAX; ++e) v[e] = ld_clamped(map, lo + e * KB + threadIdx.x, hi);
#pragma unroll
        for (int e = 0; e < ROWPASS_KMAX; ++e)
            if (lo + e * KB + threadIdx.x < hi) stage[e * KB + threadIdx.x] = v[e];
    }
    __syncthreads();
    const int32_t* row = staged ? stage + threadIdx.x * K : map + int64_t(r) * K;
    uint32_t m = 0;
    for (int k = 0; k < K; ++k) {
        const bool hit = live && row[k] >= 0;
        if (hit && k < MASK_BITS) m |= 1u << k;
        if (counts) {
            const uint64_t b = __ballot(hit);
            if ((threadIdx.x & (WAVE - 1)) == 0 && b) atomicAdd(cnt + k, int(__popcll(b)));
        }
    }
    if (keys && live) keys[r] = m;
    if (!counts) return;
    __syncthreads();
    for (int k = threadIdx.x; k < K; k += KB) counts[int64_t(k) * gridDim.x + blockIdx.x] = cnt[k];
}

// Continues a hash probe sequence past its home slot h0 (which held another key).
__device__ __noinline__ int32_t table_find_after(const uint64_t* __restrict__ table, uint32_t mask, uint32_t key,
                                                 uint32_t h0) {
    uint32_t h = (h0 + 1) & mask;
    for (uint32_t step = 1; step <= mask; ++step) {
        const uint64_t v = table[h];
        if (v == EMPTY_SLOT) return -1;
        if (uint32_t(v >> 32) == key) return int32_t(uint32_t(v));
        h = (h + 1) & mask;
    }
    return -1;
}

// Output-side map rows and their row pass in one kernel, for K <= ROWPASS_KMAX:
// one thread per output row o, whose entry k is the input row at cell
// o * stride - pad + k * dil (a submanifold map has stride 1 and pad K/2, and
// its centre entry is the row itself).  The K lookups of a row are issued
// together, so a wave has all its rows' lookups in flight at once: with the
// index grid (TBL_GRID), the K occupancy words, then the grid cells of the
// occupied neighbours; with the hash behind its bitmap filter (TBL_FILTERED),
// the K occupancy words, then the home slots of the occupied neighbours only;
// with the plain hash (TBL_HASH), all K home slots.  At load factor <= 1/4 a
// home slot answers nearly every probe (the few longer probe sequences
// continue afterwards).  Entries go to an LDS tile (row stride K words) and leave as
// coalesced row-major stores; the thread then has its row's mask (keys,
// K <= 32) and the block's per-offset hit counts (counts[k*gridDim.x +
// block]), as k_row_pass makes them.  rows < 0: M from the header (rows
// beyond the capacity read as none).
enum { TBL_HASH = 0, TBL_FILTERED = 1, TBL_GRID = 2 };

template <int TBL, bool SUBM>
__global__ __launch_bounds__(KB) void k_out_rows(const int4* __restrict__ rcoords, int32_t rows, int64_t cap, KGeom g,
                                                 const uint64_t* __restrict__ table, uint32_t mask,
                                                 const uint32_t* __restrict__ occ,
                                                 int32_t* __restrict__ nbr, uint32_t* __restrict__ keys,
                                                 int32_t* __restrict__ counts, const uint32_t* hdr,
                                                 int32_t* coord_err) {
    __shared__ uint32_t ktab[ROWPASS_KMAX];
    __shared__ int32_t cnt[ROWPASS_KMAX];
    __shared__ int32_t stage[KB * ROWPASS_KMAX];
    const int K = g.kz * g.ky * g.kx;
    const int t = threadIdx.x;
    if (t < K) {
        ktab[t] = uint32_t((t / (g.kx * g.ky)) << 6 | ((t / g.kx) % g.ky) << 3 | (t % g.kx));
        cnt[t] = 0;
    }
    __syncthreads();
    if (rows < 0) rows = rows_within(hdr, cap);
    // workgroups go to the XCDs round-robin; XCD x takes a contiguous run of
    // row blocks, so the cells that its rows look up stay in its own L2.  The
    // run is cut from the blocks that hold rows: in a grid sized by a
    // capacity above M, the blocks past M's blocks keep their own index (no
    // rows, zero counts), so that every XCD shares the rows
    const uint32_t live_blocks = (uint32_t(rows) + KB - 1) / KB;
    uint32_t lb = blockIdx.x;
    if (blockIdx.x < live_blocks) {
        const uint32_t nb = live_blocks, xc = blockIdx.x % 8u, per = nb / 8u;
        lb = xc * per + min(xc, nb % 8u) + blockIdx.x / 8u;
    }
    const int32_t row0 = int32_t(lb) * KB, i = row0 + t;
    if (coord_err && i == 0 && hdr[H_FLAGS]) atomicOr(coord_err, int32_t(hdr[H_FLAGS]));
    if (row0 >= rows) {  // uniform per block: a block past M (capacity above M) has no hits
        if (counts && t < K) counts[int64_t(t) * gridDim.x + lb] = 0;
        return;
    }
    const bool live = i < rows;
    const int4 c = rcoords[live ? i : rows - 1];
    const bool ok = live && (!SUBM || in_grid(c, g));  // output sites lie inside their grid
    constexpr bool DENSE = TBL == TBL_GRID, BITS = TBL != TBL_HASH;
    const int32_t* dense = reinterpret_cast<const int32_t*>(table);
    // 1. every lookup of the row, from valid addresses (cell 0 or its slot
    //    when the neighbour is outside the grid; such entries are -1 regardless)
    uint32_t key[ROWPASS_KMAX];
    uint64_t got[ROWPASS_KMAX];
    uint32_t inside = 0, occb = 0;  // occb (BITS): the occupancy bit of each entry's cell
    // (a SubM map's centre is looked up only with the index grid, whose
    // insert left the duplicate check to this kernel)
    if (BITS && K == 27 && g.kx == 3 && g.dx == 1) {
        // The three x-cells of each (z, y) of a 3x3x3 kernel without x
        // dilation are adjacent: one 64-bit bitmap word holds all three unless
        // the middle one sits at a word edge, where the word beside it holds
        // the third.  9 pairs of 8-byte loads instead of 27 4-byte ones, all
        // issued before any is used (the edge word is the middle cell's own
        // word when it is not needed, and clamped to the bitmap; a middle cell
        // outside the grid is clamped to its edge, and the in-grid cells are
        // placed relative to it).
        const uint64_t* occ64 = reinterpret_cast<const uint64_t*>(occ);
        const uint32_t last = uint32_t((uint64_t(g.batch) * g.Z * g.Y * g.X - 1) >> 6);
        uint64_t lo[9], hi[9];
        uint32_t rr[9];
        const int xm = c.w * g.sx - g.px + 1;  // the middle x-cell
        const int xmc = xm < 0 ? 0 : (xm >= g.X ? g.X - 1 : xm);
        int dxe[3];  // the x-cells relative to the clamped middle one
#pragma unroll
        for (int e = 0; e < 3; ++e) dxe[e] = xm - 1 + e - xmc;
#pragma unroll
        for (int q = 0; q < 9; ++q) {
            const uint32_t kk = ktab[3 * q];
            const int z = c.y * g.sz - g.pz + int(kk >> 6) * g.dz, y = c.z * g.sy - g.py + int((kk >> 3) & 7) * g.dy;
            const bool row_in = ok && (unsigned)z < (unsigned)g.Z && (unsigned)y < (unsigned)g.Y;
            const uint32_t km = row_in ? in_key(c.x, z, y, xmc, g) : 0u;
            const uint32_t w = km >> 6, r = km & 63u;
            const uint32_t w2 = r == 0u ? (w > 0u ? w - 1u : 0u) : (r == 63u ? min(w + 1u, last) : w);
            lo[q] = occ64[w];
            hi[q] = occ64[w2];
            rr[q] = r;
#pragma unroll
            for (int e = 0; e < 3; ++e) {
                const int k = 3 * q + e;
                const bool in = row_in && !(SUBM && !DENSE && k == K / 2) && (unsigned)(xm - 1 + e) < (unsigned)g.X;
                key[k] = in ? uint32_t(int(km) + dxe[e]) : 0u;
                inside |= uint32_t(in) << k;
            }
        }
#pragma unroll
        for (int q = 0; q < 9; ++q)
#pragma unroll
            for (int e = 0; e < 3; ++e) {
                // -1 .. 64 for a cell inside the grid (any bit serves the others: they are not inside)
                const int p = min(max(int(rr[q]) + dxe[e], -1), 64);
                const uint64_t b = p < 0 ? hi[q] >> 63 : (p > 63 ? hi[q] : lo[q] >> p);
                occb |= uint32_t(b & 1u) << (3 * q + e);
            }
    } else {
#pragma unroll
        for (int k = 0; k < ROWPASS_KMAX; ++k) {
            const uint32_t kk = ktab[k < K ? k : 0];
            const int z = c.y * g.sz - g.pz + int(kk >> 6) * g.dz, y = c.z * g.sy - g.py + int((kk >> 3) & 7) * g.dy,
                      x = c.w * g.sx - g.px + int(kk & 7) * g.dx;
            const bool in = ok && k < K && !(SUBM && !DENSE && k == K / 2) && (unsigned)z < (unsigned)g.Z &&
                            (unsigned)y < (unsigned)g.Y && (unsigned)x < (unsigned)g.X;
            key[k] = in ? in_key(c.x, z, y, x, g) : 0u;
            inside |= uint32_t(in) << k;
            got[k] = BITS ? uint64_t(occ[key[k] >> 5]) : table[home_slot(key[k]) & mask];
        }
        if (BITS) {
#pragma unroll
            for (int k = 0; k < ROWPASS_KMAX; ++k) occb |= ((uint32_t(got[k]) >> (key[k] & 31u)) & 1u) << k;
        }
    }
    if (DENSE) {  // grid cells of the occupied neighbours (cell 0, ignored, elsewhere)
#pragma unroll
        for (int k = 0; k < ROWPASS_KMAX; ++k) {
            const bool hit = ((inside & occb) >> k) & 1u;
            const int32_t v = dense[hit ? key[k] : 0u];
            got[k] = uint64_t(uint32_t(hit ? v : -1));
        }
    } else if (BITS) {  // home slots of the occupied neighbours (slot 0, ignored, elsewhere)
#pragma unroll
        for (int k = 0; k < ROWPASS_KMAX; ++k) {
            const bool hit = ((inside & occb) >> k) & 1u;
            const uint64_t v = table[hit ? home_slot(key[k]) & mask : 0u];
            got[k] = hit ? v : EMPTY_SLOT;
        }
    }
    // 2. resolve into LDS; hash probes that met another key finish afterwards
    uint32_t m = 0, pending = 0;
    bool dup = false;
    int32_t* srow = stage + t * K;
#pragma unroll
    for (int k = 0; k < ROWPASS_KMAX; ++k) {
        if (k >= K) continue;
        int32_t v = -1;
        if (SUBM && k == K / 2) {
            v = ok ? i : -1;
            if (DENSE && ok && int32_t(uint32_t(got[k])) != i) dup = true;
        } else if ((inside >> k) & 1u) {
            if (DENSE) {
                v = int32_t(uint32_t(got[k]));
            } else if (got[k] != EMPTY_SLOT) {
                if (uint32_t(got[k] >> 32) == key[k])
                    v = int32_t(uint32_t(got[k]));
                else
                    pending |= 1u << k;
            }
        }
        srow[k] = v;
        if (v >= 0) m |= 1u << k;
    }
    while (pending) {
        const int k = __ffs(pending) - 1;
        pending &= pending - 1;
        const uint32_t kk = ktab[k];
        const int z = c.y * g.sz - g.pz + int(kk >> 6) * g.dz, y = c.z * g.sy - g.py + int((kk >> 3) & 7) * g.dy,
                  x = c.w * g.sx - g.px + int(kk & 7) * g.dx;
        const uint32_t q = in_key(c.x, z, y, x, g);
        const int32_t v = table_find_after(table, mask, q, home_slot(q) & mask);
        srow[k] = v;
        if (v >= 0) m |= 1u << k;
    }
    if (dup && coord_err) atomicOr(coord_err, SPC_COORD_DUPLICATE);
    // 3. per-offset hit counts of the block (wave ballots into LDS)
    if (counts) {
        for (int k = 0; k < K; ++k) {
            const uint64_t b = __ballot((m >> k) & 1u);
            if ((t & (WAVE - 1)) == 0 && b) atomicAdd(cnt + k, int(__popcll(b)));
        }
    }
    if (keys && live) keys[i] = m;
    __syncthreads();
    // 4. the block's rows, row-major, coalesced
    const int64_t lo = int64_t(row0) * K, len = int64_t(min(rows, row0 + KB) - row0) * K;
#pragma unroll
    for (int e = 0; e < ROWPASS_KMAX; ++e) {
        const int j = e * KB + t;
        if (j < len) nbr[lo + j] = stage[j];
    }
    if (counts && t < K) counts[int64_t(t) * gridDim.x + lb] = cnt[t];
}

// Input-side rows of a strided map and their masks, for K <= ROWPASS_KMAX: one
// thread per input row i, whose entry k is the row of the output site
// o = (c + pad - k * dil) / stride when that division is exact on every axis
// and o lies in the output grid, else -1.  Every such site has its bitmap bit
// set, so its row is its rank: prefix[word] + the set bits below it.  Both
// words of all K entries are requested together; the rows leave through LDS
// as coalesced stores and the masks go to keys (K <= 32).  Nothing is written
// when M exceeds the capacity.
__global__ __launch_bounds__(KB) void k_in_rows(const int4* __restrict__ coords, int32_t n, int64_t cap, KGeom g,
                                                const uint32_t* __restrict__ bitmap,
                                                const uint32_t* __restrict__ prefix, int32_t* __restrict__ nbr_in,
                                                uint32_t* __restrict__ keys, const uint32_t* hdr) {
    __shared__ uint32_t ktab[ROWPASS_KMAX];
    __shared__ int32_t stage[KB * ROWPASS_KMAX];
    const int K = g.kz * g.ky * g.kx;
    const int t = threadIdx.x;
    if (t < K) ktab[t] = uint32_t((t / (g.kx * g.ky)) << 6 | ((t / g.kx) % g.ky) << 3 | (t % g.kx));
    __syncthreads();
    const int32_t row0 = blockIdx.x * KB, i = row0 + t;
    if (row0 >= n || int64_t(hdr[H_NOUT]) > cap) return;  // uniform per block
    const bool live = i < n;
    const int4 c = coords[live ? i : n - 1];
    const bool ok = live && in_grid(c, g);
    int32_t* srow = stage + t * K;
    uint32_t m = 0;
    if (K == 27 && g.kz == 3 && g.ky == 3 && g.sz >= 2 && g.sy >= 2 && g.sx >= 2 && g.dz == 1 && g.dy == 1 &&
        g.dx == 1) {
        // Stride >= 2 with 3 offsets per axis and no dilation: at most 2
        // offsets per axis reach an output site (their c + pad - k span less
        // than 2 strides), so at most 8 of the 27 entries exist.  Their sites
        // are found per axis, and only those 8 combinations load a bitmap
        // word and a prefix (invalid ones from word 0); the rest of the row
        // is -1.
        int ka[3][2], oa[3][2], na[3];
        const int cc[3] = {c.y, c.z, c.w}, pp[3] = {g.pz, g.py, g.px}, dd[3] = {g.dz, g.dy, g.dx},
                  ss[3] = {g.sz, g.sy, g.sx}, ext[3] = {g.oz, g.oy, g.ox};
        const uint64_t ms[3] = {g.msz, g.msy, g.msx};
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            na[a] = 0;
            ka[a][0] = ka[a][1] = 0;
            oa[a][0] = oa[a][1] = 0;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int num = cc[a] + pp[a] - k * dd[a];
                const int o = num >= 0 ? int(qdiv(uint32_t(num), ms[a])) : -1;
                const bool hit = o >= 0 && o * ss[a] == num && o < ext[a];
                if (hit && na[a] < 2) {
                    ka[a][na[a]] = k;
                    oa[a][na[a]] = o;
                    ++na[a];
                }
            }
        }
        uint32_t bits8[8], pre8[8], pos8[8];
        bool in8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int iz = q >> 2, iy = (q >> 1) & 1, ix = q & 1;
            in8[q] = ok && iz < na[0] && iy < na[1] && ix < na[2];
            const uint32_t key = in8[q] ? out_key(c.x, oa[0][iz], oa[1][iy], oa[2][ix], g) : 0u;
            pos8[q] = key & 31u;
            bits8[q] = bitmap[key >> 5];
            pre8[q] = prefix[key >> 5];
        }
#pragma unroll
        for (int k = 0; k < 27; ++k) srow[k] = -1;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (!in8[q]) continue;
            const int k = (ka[0][q >> 2] * 3 + ka[1][(q >> 1) & 1]) * 3 + ka[2][q & 1];
            srow[k] = int32_t(pre8[q] + __popc(bits8[q] & ((1u << pos8[q]) - 1u)));
            m |= 1u << k;
        }
    } else {
    uint32_t bitpos[ROWPASS_KMAX], bits[ROWPASS_KMAX], pre[ROWPASS_KMAX];
    uint32_t valid = 0;
#pragma unroll
    for (int k = 0; k < ROWPASS_KMAX; ++k) {
        const uint32_t kk = ktab[k < K ? k : 0];
        const int nz = c.y + g.pz - int(kk >> 6) * g.dz, ny = c.z + g.py - int((kk >> 3) & 7) * g.dy,
                  nx = c.w + g.px - int(kk & 7) * g.dx;
        const int oz = nz >= 0 ? int(qdiv(uint32_t(nz), g.msz)) : -1;
        const int oy = ny >= 0 ? int(qdiv(uint32_t(ny), g.msy)) : -1;
        const int ox = nx >= 0 ? int(qdiv(uint32_t(nx), g.msx)) : -1;
        const bool in = ok && k < K && oz >= 0 && oy >= 0 && ox >= 0 && oz * g.sz == nz && oy * g.sy == ny &&
                        ox * g.sx == nx && oz < g.oz && oy < g.oy && ox < g.ox;
        const uint32_t key = in ? out_key(c.x, oz, oy, ox, g) : 0u;
        valid |= uint32_t(in) << k;
        bitpos[k] = key & 31u;
        bits[k] = bitmap[key >> 5];
        pre[k] = prefix[key >> 5];
    }
#pragma unroll
    for (int k = 0; k < ROWPASS_KMAX; ++k) {
        if (k >= K) continue;
        const bool in = (valid >> k) & 1u;
        srow[k] = in ? int32_t(pre[k] + __popc(bits[k] & ((1u << bitpos[k]) - 1u))) : -1;
        if (in) m |= 1u << k;
    }
    }
    if (keys && live) keys[i] = m;
    __syncthreads();
    const int64_t lo = int64_t(row0) * K, len = int64_t(min(n, row0 + KB) - row0) * K;
#pragma unroll
    for (int e = 0; e < ROWPASS_KMAX; ++e) {
        const int j = e * KB + t;
        if (j < len) nbr_in[lo + j] = stage[j];
    }
}

// Ordered compaction of one block of map rows into the CSR pair lists: for
// each offset k, the block's hits go to the scanned offset offs[k*nblk +
// block] in ascending row order.  With masks (K <= ROWPASS_KMAX) the ranks of
// all offsets come from one ballot each and a single barrier, and offs holds
// per-offset scans whose totals are at hdr[H_TOT + k]: the block adds their
// prefix, and block 0 writes the CSR offsets to pair_ptr.  Otherwise offs is
// one scan of the whole matrix and there is one block scan per offset.
// rows < 0: read M from the header.
__global__ __launch_bounds__(KB) void k_compact_pairs(const int32_t* __restrict__ map, int32_t rows, int K,
                                                      int64_t cap, const uint32_t* hdr,
                                                      const uint32_t* __restrict__ masks,
                                                      const int32_t* __restrict__ offs,
                                                      int32_t* __restrict__ pair_in,
                                                      int32_t* __restrict__ pair_out, int32_t* pair_ptr) {
    __shared__ int waves[KB / WAVE];
    __shared__ int wcnt[ROWPASS_KMAX][KB / WAVE];
    if (rows < 0) rows = rows_within(hdr, cap);
    const int32_t o = blockIdx.x * KB + threadIdx.x;
    const bool live = o < rows;
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    if (masks) {
        __shared__ int32_t stage[KB * ROWPASS_KMAX];
        __shared__ int32_t soff[ROWPASS_KMAX];
        const uint32_t m = live ? masks[o] : 0u;
        const uint64_t lt = (1ull << lane) - 1ull;
        const int32_t row0 = blockIdx.x * KB;
        if (wave == 0) {  // this block's slot per offset: the offsets before it, then the blocks before it
            const int32_t tk = lane < K ? int32_t(hdr[H_TOT + lane]) : 0;
            int incl = tk;
            for (int off = 1; off < WAVE; off <<= 1) {
                const int u = __shfl_up(incl, off);
                if (lane >= off) incl += u;
            }
            if (lane < K) soff[lane] = incl - tk + offs[int64_t(lane) * gridDim.x + blockIdx.x];
            if (blockIdx.x == 0 && lane <= K) pair_ptr[lane] = incl - tk;
        }
        if (row0 < rows) {
            const int64_t lo = int64_t(row0) * K, hi = int64_t(min(rows, row0 + KB)) * K;
            int32_t v[ROWPASS_KMAX];
#pragma unroll
            for (int e = 0; e < ROWPASS_KMAX; ++e) v[e] = ld_clamped(map, lo + e * KB + threadIdx.x, hi);
#pragma unroll
            for (int e = 0; e < ROWPASS_KMAX; ++e)
                if (lo + e * KB + threadIdx.x < hi) stage[e * KB + threadIdx.x] = v[e];
        }
        for (int k = 0; k < K; ++k) {
            const uint64_t b = __ballot((m >> k) & 1u);
            if (lane == 0) wcnt[k][wave] = __popcll(b);
        }
        __syncthreads();
        for (int k = 0; k < K; ++k) {  // uniform loop: every lane takes part in the ballots
            const bool hit = (m >> k) & 1u;
            const uint64_t b = __ballot(hit);
            if (!hit) continue;
            int before = 0;
            for (int w = 0; w < wave; ++w) before += wcnt[k][w];
            const int64_t at = int64_t(soff[k]) + before + __popcll(b & lt);
            pair_in[at] = stage[threadIdx.x * K + k];
            pair_out[at] = o;
        }
        return;
    }
    for (int k = 0; k < K; ++k) {
        const int32_t v = live ? map[int64_t(o) * K + k] : -1;
        int total;
        const int pos = block_exclusive_scan<KB>(v >= 0 ? 1 : 0, waves, total);
        if (v >= 0) {
            const int64_t at = int64_t(offs[int64_t(k) * gridDim.x + blockIdx.x]) + pos;
            pair_in[at] = v;
            pair_out[at] = o;
        }
    }
}

// Identity order (used when K > 32 leaves no mask to sort by).
__global__ void k_iota(int32_t* __restrict__ out, int32_t rows, int64_t cap, const uint32_t* hdr) {
    if (rows < 0) rows = rows_within(hdr, cap);
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < rows; i += stride) out[i] = int32_t(i);
}

// ---------------------------------------------------------------- host side

struct Plan {
    KGeom g;
    int K;
    int64_t n;
    uint32_t cap_log2;
    int64_t cap;                 // table slots
    int64_t out_vol;             // strided output grid volume
    int64_t nwords;              // bitmap words (multiple of WORDS_PER_THREAD)
    bool bytemap;                // strided output sites marked in a byte map (32 bytes per bitmap word)
    int64_t m_max;               // upper bound of the output row count
    int64_t rows_max;            // max(n, m_max)
    int64_t cblk;                // count-matrix blocks per offset
    int64_t rblk;                // radix blocks
    int64_t bm_blocks;           // bitmap count/emit blocks
    // workspace offsets
    int64_t rgroups;             // radix block groups
    int64_t occ_words;           // input occupancy bitmap words (multiple of 4)
    size_t off_table, off_occ, off_counts, off_bitmap, off_sites, off_prefix, off_bsums, off_masks, off_sort, off_gsum,
        off_gtot, total;
    size_t sort_slot_bytes;      // per sort: keys x2, values x2, histogram matrix
};

spc_status make_plan(const spc_geom* gp, int64_t n_in, Plan& p) {
    if (!gp) return fail(SPC_ERR_ARG, "geometry pointer is NULL");
    const spc_geom& g = *gp;
    if (n_in < 0 || n_in >= (int64_t(1) << 31)) return fail(SPC_ERR_ARG, "n_in=%lld out of range", (long long)n_in);
    if (g.batch <= 0) return fail(SPC_ERR_ARG, "batch=%d must be positive", g.batch);
    for (int a = 0; a < 3; ++a) {
        if (g.shape[a] <= 0) return fail(SPC_ERR_ARG, "shape[%d]=%d must be positive", a, g.shape[a]);
        if (g.ksize[a] <= 0 || g.ksize[a] > 7)
            return fail(SPC_ERR_UNSUPPORTED, "ksize[%d]=%d: supported kernel sizes are 1..7", a, g.ksize[a]);
        if (g.subm && g.ksize[a] % 2 == 0)
            return fail(SPC_ERR_ARG, "submanifold ksize[%d]=%d must be odd", a, g.ksize[a]);
        if (!g.subm && (g.stride[a] <= 0 || g.dil[a] <= 0 || g.pad[a] < 0))
            return fail(SPC_ERR_ARG, "axis %d: stride=%d dil=%d pad=%d invalid", a, g.stride[a], g.dil[a], g.pad[a]);
    }
    KGeom& k = p.g;
    k.batch = g.batch;
    k.Z = g.shape[0]; k.Y = g.shape[1]; k.X = g.shape[2];
    k.kz = g.ksize[0]; k.ky = g.ksize[1]; k.kx = g.ksize[2];
    if (g.subm) {
        k.sz = k.sy = k.sx = 1;
        k.pz = k.kz / 2; k.py = k.ky / 2; k.px = k.kx / 2;
        k.dz = k.dy = k.dx = 1;
        k.oz = k.Z; k.oy = k.Y; k.ox = k.X;
    } else {
        k.sz = g.stride[0]; k.sy = g.stride[1]; k.sx = g.stride[2];
        k.pz = g.pad[0]; k.py = g.pad[1]; k.px = g.pad[2];
        k.dz = g.dil[0]; k.dy = g.dil[1]; k.dx = g.dil[2];
        int32_t os[3];
        spc_out_shape(gp, os);
        k.oz = os[0] > 0 ? os[0] : 0;
        k.oy = os[1] > 0 ? os[1] : 0;
        k.ox = os[2] > 0 ? os[2] : 0;
    }
    // an input reaches at most ksize <= 7 outputs per axis (k_insert keeps 8 slots)
    p.K = k.kz * k.ky * k.kx;
    k.mK = recip64(uint64_t(p.K));
    k.msz = recip64(uint64_t(k.sz));
    k.msy = recip64(uint64_t(k.sy));
    k.msx = recip64(uint64_t(k.sx));
    k.mox = recip64(uint64_t(k.ox));
    k.mplane = recip64(uint64_t(k.oy) * uint64_t(k.ox));
    k.mvol = recip64(uint64_t(k.oz) * uint64_t(k.oy) * uint64_t(k.ox));
    const uint64_t in_vol = uint64_t(g.batch) * k.Z * k.Y * k.X;
    if (in_vol >= (uint64_t(1) << 32))
        return fail(SPC_ERR_UNSUPPORTED, "batch*Z*Y*X = %llu must be below 2^32", (unsigned long long)in_vol);
    p.out_vol = g.subm ? 0 : int64_t(uint64_t(g.batch) * k.oz * k.oy * k.ox);
    if (uint64_t(p.out_vol) >= (uint64_t(1) << 32))
        return fail(SPC_ERR_UNSUPPORTED, "output grid volume %lld must be below 2^32", (long long)p.out_vol);
    if (int64_t(p.K) * n_in >= (int64_t(1) << 31))
        return fail(SPC_ERR_UNSUPPORTED, "K*n_in=%lld must be below 2^31", (long long)(int64_t(p.K) * n_in));
    p.n = n_in;
    // The input table.  SPC_TABLE_HASH: the hash, whose load factor <= 1/4
    // keeps unsuccessful probes (most of them) near one load.
    // SPC_TABLE_GRID: an occupancy bitmap, one bit per cell, cleared per call,
    // and beside it the index grid, one int32 row per cell.  An insert sets
    // its bit with one atomic OR, whose old value flags a duplicate, and
    // stores its row in the grid; the grid is read only where the bitmap says
    // occupied, so it is never cleared.  A lookup is a bitmap word and, for an
    // occupied cell, one grid load.  The table region is cap 8-byte words.
    // The hash gets the occupancy bitmap beside it as an exact filter when the
    // bitmap is small next to the rows (at most 1 KiB per row, at most 1 GiB):
    // most of a sparse scene's K lookups per row find an empty cell, and then
    // cost a bitmap word (neighbouring cells share words) instead of a hash
    // probe at a random slot; the hash is probed for occupied cells only.
    if (g.table != SPC_TABLE_HASH && g.table != SPC_TABLE_GRID)
        return fail(SPC_ERR_ARG, "table=%d must be SPC_TABLE_HASH or SPC_TABLE_GRID", g.table);
    k.dense = g.table == SPC_TABLE_GRID;
    k.occ = k.dense || (in_vol <= OCC_FILTER_CELLS_PER_ROW * uint64_t(std::max<int64_t>(n_in, 1)) &&
                        in_vol / 8 <= OCC_FILTER_MAX_BYTES);
    p.occ_words = k.occ ? int64_t(ceil_div(int64_t(in_vol), 128) * 4) : 0;
    p.cap_log2 = 6;
    while ((int64_t(1) << p.cap_log2) < 4 * n_in) ++p.cap_log2;
    p.cap = k.dense ? int64_t((in_vol + 1) / 2) : int64_t(1) << p.cap_log2;
    const int64_t wpb = int64_t(KB) * WORDS_PER_THREAD;
    p.nwords = g.subm ? 0 : std::max<int64_t>(wpb, ceil_div(ceil_div(p.out_vol, 32), wpb) * wpb);
    p.bm_blocks = p.nwords / wpb;
    // Strided output sites: many input rows reach each site (up to 8 for
    // k3 s2), so atomic ORs on a bitmap word contend.  A byte per site takes
    // plain stores instead (idempotent, so concurrent rows need no atomics),
    // and the count kernel packs the bytes into the bitmap.  That costs
    // clearing and reading a byte per site, and scattered byte stores into a
    // map larger than the caches are slow: it pays on output grids that are
    // dense next to the rows (shell sets: 4 sites per input row, strided map
    // 236 -> 205 us), not on sparse ones (LiDAR scene: 197 sites per row, no
    // gain).
    p.bytemap = !g.subm && uint64_t(p.nwords) * 32 <= BYTEMAP_MAX_SITES &&
                uint64_t(p.nwords) * 32 <= BYTEMAP_SITES_PER_ROW * uint64_t(std::max<int64_t>(n_in, 1));
    p.m_max = g.subm ? n_in : std::min<int64_t>(int64_t(p.K) * n_in, p.out_vol);
    p.rows_max = std::max(n_in, p.m_max);
    p.cblk = ceil_div(p.rows_max, KB);
    p.rblk = ceil_div(p.rows_max, RS_TILE);
    size_t off = 256;
    p.off_table = off;   off = align_up(off + size_t(p.cap) * 8, 256);
    p.off_occ = off;     off = align_up(off + size_t(p.occ_words) * 4, 256);
    p.off_counts = off;  off = align_up(off + size_t(p.K) * p.cblk * 4, 256);
    p.off_bitmap = off;  off = align_up(off + size_t(p.nwords) * 4, 256);
    p.off_sites = off;   off = align_up(off + (p.bytemap ? size_t(p.nwords) * 32 : 0), 256);
    p.off_prefix = off;  off = align_up(off + size_t(p.nwords) * 4, 256);
    p.off_bsums = off;   off = align_up(off + size_t(p.bm_blocks) * 4 + 4, 256);
    p.off_masks = off;   off = align_up(off + size_t(p.rows_max) * 4 * 2, 256);   // neighbour masks, per sort
    p.sort_slot_bytes = align_up(size_t(p.rows_max) * 4 * 4 + size_t(RS_BINS) * p.rblk * 4, 256);
    p.off_sort = off;    off += 2 * p.sort_slot_bytes;                            // sort buffers, per sort
    p.rgroups = ceil_div(p.rblk, RS_GROUP);
    p.off_gsum = off;    off = align_up(off + size_t(2 * RS_MAX_PASSES) * RS_BINS * p.rgroups * 4, 256);
    p.off_gtot = off;    off = align_up(off + size_t(2 * RS_MAX_PASSES) * RS_BINS * 4, 256);     // spine totals
    p.total = off;
    return SPC_OK;
}

inline unsigned grid_for(int64_t work, int64_t per_block, int64_t cap = 1 << 16) {
    int64_t b = ceil_div(std::max<int64_t>(work, 1), per_block);
    return unsigned(std::min<int64_t>(std::max<int64_t>(b, 1), cap));
}

// Buffers of one radix sort (each of the two sorts of a strided call has its
// own, so the input side's masks stay intact while the output side sorts).
struct SortBuf {
    uint32_t* keys[2];
    int32_t* vals[2];
    int32_t* hist;
};

struct Scratch {
    uint32_t* hdr;
    int32_t* counts;
    uint32_t* mask[2];           // neighbour masks of the rows, per sort slot
    SortBuf sort[2];
    int32_t* gsum;               // [2 sorts][RS_MAX_PASSES][RS_BINS][groups], zeroed by k_clear
    int32_t* gtot;               // [2 sorts][RS_MAX_PASSES][RS_BINS] spine totals (written before read)
};

// Row pass: masks into keys (K <= 32, NULL ok) and per-block counts (NULL ok).
spc_status row_pass(const Plan& p, const int32_t* map, int32_t rows_dev, int64_t rows_cap, int64_t cap,
                    const Scratch& s, uint32_t* keys, int32_t* counts, hipStream_t stream) {
    const int64_t blk = ceil_div(rows_cap, KB);
    if (blk == 0) return SPC_OK;
    hipLaunchKernelGGL(k_row_pass, dim3(unsigned(blk)), dim3(KB), 0, stream, map, rows_dev,
                       p.K, cap, s.hdr, p.K <= MASK_BITS ? keys : nullptr, counts);
    SPC_LAUNCHED("k_row_pass");
    return SPC_OK;
}

// Stable LSD radix sort of the rows of `map` by neighbour mask into `order`
// (the identity for K > 32), with sort slot `slot`'s buffers and group sums.
// masks_ready: s.mask[slot] already holds the masks (else a row pass makes
// them).  The masks are only read, so a concurrent pair compaction may read
// them too.  rows_dev < 0 means M from the header; grids are sized for
// rows_cap rows.
// One processing order to build: the rows of `map` (rows_dev < 0: M from the
// header; grids sized for rows_cap rows) sorted by neighbour mask into
// `order`, with sort slot `slot`'s buffers; masks_ready: s.mask[slot] already
// holds the masks (else a row pass makes them).
struct OrderJob {
    const int32_t* map;
    int32_t rows_dev;
    int64_t rows_cap, cap;
    bool masks_ready;
    int slot;
    int32_t* order;
};

// Stable LSD radix sorts of up to two orders (the identity for K > 32).  Two
// orders share each pass's launches: blocks [0, nb0) sort the first, the rest
// the second.  The masks are only read, so a pair compaction may read them
// afterwards.
spc_status sort_orders(const Plan& p, const Scratch& s, const OrderJob* jobs, int count, hipStream_t stream) {
    const int K = p.K;
    const OrderJob* live[2] = {nullptr, nullptr};
    int nl = 0;
    for (int i = 0; i < count; ++i) {
        const OrderJob& o = jobs[i];
        if (K > MASK_BITS) {
            hipLaunchKernelGGL(k_iota, dim3(grid_for(o.rows_cap, KB, 4096)), dim3(KB), 0, stream, o.order, o.rows_dev,
                               o.cap, s.hdr);
            SPC_LAUNCHED("k_iota");
            continue;
        }
        if (o.rows_cap == 0) continue;
        if (!o.masks_ready) {
            spc_status st = row_pass(p, o.map, o.rows_dev, o.rows_cap, o.cap, s, s.mask[o.slot], nullptr, stream);
            if (st != SPC_OK) return st;
        }
        live[nl++] = &o;
    }
    if (nl == 0) return SPC_OK;
    const int passes = (K + RS_BITS - 1) / RS_BITS;
    RsPass P{};
    for (int i = 0; i < nl; ++i) {
        RsJob& J = P.job[i];
        J.keys_in = s.mask[live[i]->slot];
        J.vals_in = nullptr;
        J.n_dev = s.hdr + H_NOUT;
        J.cap = live[i]->cap;
        J.rows = live[i]->rows_dev;
        J.nb = int(ceil_div(live[i]->rows_cap, RS_TILE));
        J.ng = int(ceil_div(J.nb, RS_GROUP));
        J.hist = s.sort[live[i]->slot].hist;
    }
    const unsigned blocks = unsigned(P.job[0].nb + P.job[1].nb);
    for (int pass = 0; pass < passes; ++pass) {
        P.shift = RS_BITS * pass;
        const bool last = pass + 1 == passes;
        for (int i = 0; i < nl; ++i) {
            const int slot = live[i]->slot;
            const SortBuf& sb = s.sort[slot];
            P.job[i].gsum = s.gsum + (int64_t(slot) * RS_MAX_PASSES + pass) * RS_BINS * p.rgroups;
            // many groups (a sort sized by a large capacity): one spine launch
            // scans them, instead of every scatter block reading them all
            P.job[i].gtot = P.job[i].ng > RS_SPINE_GROUPS
                                ? s.gtot + (int64_t(slot) * RS_MAX_PASSES + pass) * RS_BINS
                                : nullptr;
            P.job[i].keys_out = sb.keys[pass & 1];
            P.job[i].vals_out = last ? live[i]->order : sb.vals[pass & 1];
        }
        hipLaunchKernelGGL(k_rs_hist, dim3(blocks), dim3(RS_THREADS), 0, stream, P);
        SPC_LAUNCHED("k_rs_hist");
        if (P.job[0].gtot || P.job[1].gtot) {
            hipLaunchKernelGGL(k_rs_spine, dim3(2 * RS_BINS / 4), dim3(256), 0, stream, P);
            SPC_LAUNCHED("k_rs_spine");
        }
        hipLaunchKernelGGL(k_rs_scatter, dim3(blocks), dim3(RS_THREADS), 0, stream, P);
        SPC_LAUNCHED("k_rs_scatter");
        for (int i = 0; i < nl; ++i) {
            P.job[i].keys_in = P.job[i].keys_out;
            P.job[i].vals_in = P.job[i].vals_out;
        }
    }
    return SPC_OK;
}

spc_status sort_rows(const Plan& p, const int32_t* map, int32_t rows_dev, int64_t rows_cap, int64_t cap,
                     const Scratch& s, bool masks_ready, int slot, int32_t* order, hipStream_t stream) {
    const OrderJob o{map, rows_dev, rows_cap, cap, masks_ready, slot, order};
    return sort_orders(p, s, &o, 1, stream);
}

// Pinned host words and an event per host thread and device: a strided call
// copies M and the coordinate flags there as soon as they are known and waits
// for that copy only, so the host returns while the rest of the map is built.
struct HostCount {
    hipEvent_t ev = nullptr;
    uint32_t* words = nullptr;
};

// The row count of a call whose count the host knows (SubM: the input rows):
// to the host word, or, for the call that does not wait, to the device word.
spc_status publish_known(int64_t n, int64_t* n_out, int32_t* n_out_dev, hipStream_t stream) {
    if (!n_out_dev) {
        *n_out = n;
        return SPC_OK;
    }
    hipLaunchKernelGGL(k_publish_count, dim3(1), dim3(WAVE), 0, stream, static_cast<const uint32_t*>(nullptr),
                       int32_t(n), n_out_dev);
    SPC_LAUNCHED("k_publish_count");
    return SPC_OK;
}

spc_status host_count_for_device(HostCount** out) {
    static thread_local HostCount hcs[64];
    int dev = 0;
    SPC_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return fail(SPC_ERR_UNSUPPORTED, "device %d", dev);
    HostCount& h = hcs[dev];
    if (!h.ev) {
        SPC_HIP(hipHostMalloc(reinterpret_cast<void**>(&h.words), 64, hipHostMallocDefault));
        SPC_HIP(hipEventCreateWithFlags(&h.ev, hipEventDisableTiming));
    }
    *out = &h;
    return SPC_OK;
}

// Scan and ordered compaction of a map into CSR pairs, from the counts (and,
// for K <= 27, the masks in s.mask[0]) of a row pass already enqueued.
spc_status map_pairs(const Plan& p, const int32_t* map, int32_t rows_dev, int64_t rows_cap, int64_t cap,
                     const Scratch& s, int32_t* pair_ptr, int32_t* pair_in, int32_t* pair_out, hipStream_t stream) {
    const int64_t blk = ceil_div(rows_cap, KB);
    const bool masked = p.K <= ROWPASS_KMAX && blk > 0;
    if (masked) {  // each offset's row of the count matrix scanned by its own workgroup
        hipLaunchKernelGGL(k_scan, dim3(unsigned(p.K)), dim3(SCAN_THREADS), 0, stream, s.counts, blk,
                           (int32_t*)nullptr, 0, int64_t(0), s.hdr + H_TOT);
    } else {
        hipLaunchKernelGGL(k_scan, dim3(1), dim3(SCAN_THREADS), 0, stream, s.counts, int64_t(p.K) * blk, pair_ptr,
                           p.K, blk, (uint32_t*)nullptr);
    }
    SPC_LAUNCHED("k_scan");
    if (blk > 0) {
        hipLaunchKernelGGL(k_compact_pairs, dim3(unsigned(blk)), dim3(KB), 0, stream, map, rows_dev, p.K, cap, s.hdr,
                           masked ? s.mask[0] : nullptr, s.counts, pair_in, pair_out, pair_ptr);
        SPC_LAUNCHED("k_compact_pairs");
    }
    return SPC_OK;
}

}  // namespace
}  // namespace spc

using namespace spc;

extern "C" spc_status spc_out_shape(const spc_geom* g, int32_t out_shape[3]) {
    clear_error();
    if (!g || !out_shape) return fail(SPC_ERR_ARG, "NULL argument");
    for (int a = 0; a < 3; ++a) {
        if (g->subm) {
            out_shape[a] = g->shape[a];
            continue;
        }
        if (g->stride[a] <= 0) return fail(SPC_ERR_ARG, "stride[%d]=%d must be positive", a, g->stride[a]);
        const int64_t num = int64_t(g->shape[a]) + 2 * int64_t(g->pad[a]) -
                            int64_t(g->dil[a]) * (g->ksize[a] - 1) - 1;
        // floor division (num may be negative)
        const int64_t q = num >= 0 ? num / g->stride[a] : -((-num + g->stride[a] - 1) / g->stride[a]);
        out_shape[a] = int32_t(q + 1);
    }
    return SPC_OK;
}

extern "C" spc_status spc_kmap_workspace(const spc_geom* g, int64_t n_in, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(SPC_ERR_ARG, "bytes is NULL");
    Plan p;
    spc_status st = make_plan(g, n_in, p);
    if (st != SPC_OK) return st;
    *bytes = p.total;
    return SPC_OK;
}

namespace spc {
namespace {

// spc_build_kmap (n_out on the host: the strided form waits for its count)
// and spc_build_kmap_async (n_out_dev in device memory: nothing waits).
spc_status build_kmap(const spc_geom* gp, const int32_t* coords, int64_t n_in, int32_t* out_coords, int64_t out_cap,
                      int64_t* n_out, int32_t* n_out_dev, int32_t* nbr, int32_t* nbr_in, int32_t* pair_ptr,
                      int32_t* pair_in, int32_t* pair_out, int64_t pair_cap, int32_t* order, int32_t* order_in,
                      int32_t* coord_err, void* ws, size_t ws_bytes, hipStream_t stream) {
    Plan p;
    spc_status st = make_plan(gp, n_in, p);
    if (st != SPC_OK) return st;
    const bool subm = gp->subm != 0;
    const bool wait = n_out_dev == nullptr;
    const bool strided_count_only = !subm && out_coords == nullptr;
    if (wait && !n_out) return fail(SPC_ERR_ARG, "n_out is NULL");
    if (!wait && strided_count_only) return fail(SPC_ERR_ARG, "the call that does not wait needs out_coords");
    if (!wait && !aligned16(n_out_dev)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    if (n_in > 0 && !coords) return fail(SPC_ERR_ARG, "coords is NULL");
    if (!ws) return fail(SPC_ERR_ARG, "workspace is NULL");
    if (ws_bytes < p.total) return fail(SPC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, p.total);
    const bool pairs = pair_ptr || pair_in || pair_out;
    if (pairs && !(pair_ptr && pair_in && pair_out)) return fail(SPC_ERR_ARG, "pair_ptr/pair_in/pair_out must be all set or all NULL");
    if (pairs && pair_cap < int64_t(p.K) * n_in) return fail(SPC_ERR_ARG, "pair_cap=%lld < K*n_in=%lld", (long long)pair_cap, (long long)(int64_t(p.K) * n_in));
    if (!strided_count_only && !nbr) return fail(SPC_ERR_ARG, "nbr is NULL");
    if (!subm && !strided_count_only && out_cap < 0) return fail(SPC_ERR_ARG, "out_cap < 0");
    if (subm && order_in) return fail(SPC_ERR_ARG, "order_in is for strided maps only");
    if (order_in && !nbr_in && n_in > 0) return fail(SPC_ERR_ARG, "order_in needs nbr_in");
    const void* ptrs[] = {coords, out_coords, nbr, nbr_in, pair_ptr, pair_in, pair_out, order, order_in, coord_err, ws};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");

    char* base = static_cast<char*>(ws);
    Scratch s;
    s.hdr = reinterpret_cast<uint32_t*>(base);
    s.counts = reinterpret_cast<int32_t*>(base + p.off_counts);
    s.mask[0] = reinterpret_cast<uint32_t*>(base + p.off_masks);
    s.mask[1] = s.mask[0] + p.rows_max;
    for (int q = 0; q < 2; ++q) {
        char* b = base + p.off_sort + q * p.sort_slot_bytes;
        SortBuf& sb = s.sort[q];
        sb.keys[0] = reinterpret_cast<uint32_t*>(b);
        sb.keys[1] = sb.keys[0] + p.rows_max;
        sb.vals[0] = reinterpret_cast<int32_t*>(sb.keys[1] + p.rows_max);
        sb.vals[1] = sb.vals[0] + p.rows_max;
        sb.hist = sb.vals[1] + p.rows_max;
    }
    s.gsum = reinterpret_cast<int32_t*>(base + p.off_gsum);
    s.gtot = reinterpret_cast<int32_t*>(base + p.off_gtot);
    uint64_t* table = reinterpret_cast<uint64_t*>(base + p.off_table);
    uint32_t* occ = reinterpret_cast<uint32_t*>(base + p.off_occ);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + p.off_bitmap);
    uint8_t* sites = p.bytemap ? reinterpret_cast<uint8_t*>(base + p.off_sites) : nullptr;
    uint32_t* prefix = reinterpret_cast<uint32_t*>(base + p.off_prefix);
    int32_t* bsums = reinterpret_cast<int32_t*>(base + p.off_bsums);
    const int4* c4 = reinterpret_cast<const int4*>(coords);
    const int32_t n = int32_t(n_in);
    const uint32_t mask = uint32_t(p.cap - 1);
    const int32_t nblk = int32_t(ceil_div(n, KB));
    const int64_t entries = int64_t(n) * p.K;

    const int64_t nzero = (order || order_in) ? int64_t(2 * RS_MAX_PASSES) * RS_BINS * p.rgroups : 0;
    const int64_t fill = p.g.dense ? 0 : p.cap;   // hash slots to mark empty (the index grid is never cleared)
    // the byte map is cleared in place of the bitmap, which the count kernel then writes whole
    uint32_t* clear_bits = sites ? reinterpret_cast<uint32_t*>(sites) : bitmap;
    const int64_t clear_words = sites ? p.nwords * 8 : p.nwords;
    hipLaunchKernelGGL(k_clear, dim3(grid_for(std::max({fill / 2, clear_words / 4, p.occ_words / 4, nzero / 4}), KB, 4096)),
                       dim3(KB), 0, stream, table, fill, clear_bits, clear_words, occ, p.occ_words, s.hdr, coord_err,
                       s.gsum, nzero);
    SPC_LAUNCHED("k_clear");
    if (n > 0) {
        if (subm)
            hipLaunchKernelGGL(k_insert<false>, dim3(nblk), dim3(KB), 0, stream, c4, n, p.g, table, mask, occ, bitmap,
                               (uint8_t*)nullptr, s.hdr);
        else
            hipLaunchKernelGGL(k_insert<true>, dim3(nblk), dim3(KB), 0, stream, c4, n, p.g, table, mask, occ, bitmap,
                               sites, s.hdr);
        SPC_LAUNCHED("k_insert");
    }

    if (subm && p.K <= ROWPASS_KMAX) {
        // probes, masks and counts in one pass over the rows
        auto rows_kernel = p.g.dense ? k_out_rows<TBL_GRID, true>
                                     : p.g.occ ? k_out_rows<TBL_FILTERED, true> : k_out_rows<TBL_HASH, true>;
        hipLaunchKernelGGL(rows_kernel, dim3(unsigned(std::max(nblk, 1))), dim3(KB), 0, stream, c4, n, int64_t(n), p.g,
                           table, mask,
                           occ, nbr, (pairs || order) ? s.mask[0] : nullptr, pairs ? s.counts : nullptr, s.hdr,
                           coord_err);
        SPC_LAUNCHED("k_out_rows");
        if (pairs) {
            st = map_pairs(p, nbr, n, n, n, s, pair_ptr, pair_in, pair_out, stream);
            if (st != SPC_OK) return st;
        }
        if (order) {
            st = sort_rows(p, nbr, n, n, n, s, true, 0, order, stream);
            if (st != SPC_OK) return st;
        }
        return publish_known(n_in, n_out, n_out_dev, stream);
    }
    if (subm) {
        hipLaunchKernelGGL(k_subm_probe, dim3(unsigned(std::max<int64_t>(ceil_div(entries, KB), 1))), dim3(KB), 0,
                           stream, c4, n, p.g, table, mask, occ, nbr, s.hdr, coord_err);
        SPC_LAUNCHED("k_subm_probe");
        if (pairs || order) {
            // one row pass: the masks (for the order and the compaction) and the counts
            st = row_pass(p, nbr, n, n, n, s, s.mask[0], pairs ? s.counts : nullptr, stream);
            if (st != SPC_OK) return st;
        }
        if (pairs) {
            st = map_pairs(p, nbr, n, n, n, s, pair_ptr, pair_in, pair_out, stream);
            if (st != SPC_OK) return st;
        }
        if (order) {
            st = sort_rows(p, nbr, n, n, n, s, true, 0, order, stream);
            if (st != SPC_OK) return st;
        }
        return publish_known(n_in, n_out, n_out_dev, stream);
    }

    // strided: output sites into the bitmap, then count them (total -> hdr,
    // by atomics; the per-block counts are scanned separately only for large
    // bitmaps, else each emit block sums the counts before it)
    hipLaunchKernelGGL(k_bitmap_count, dim3(unsigned(p.bm_blocks)), dim3(KB), 0, stream, bitmap, p.nwords, sites,
                       bsums, s.hdr + H_NOUT);
    SPC_LAUNCHED("k_bitmap_count");
    const bool scanned = p.bm_blocks > EMIT_SUM_BLOCKS;
    if (scanned) {
        hipLaunchKernelGGL(k_scan, dim3(1), dim3(SCAN_THREADS), 0, stream, bsums, p.bm_blocks, (int32_t*)nullptr, 0,
                           int64_t(0), (uint32_t*)nullptr);
        SPC_LAUNCHED("k_scan");
    }
    // M and the flags are final here: their copy goes first, and the host waits
    // for it alone once everything else is enqueued
    HostCount* hc = nullptr;
    if (wait) {
        if ((st = host_count_for_device(&hc)) != SPC_OK) return st;
        SPC_HIP(hipMemcpyAsync(hc->words, s.hdr, 2 * sizeof(uint32_t), hipMemcpyDeviceToHost, stream));
        SPC_HIP(hipEventRecord(hc->ev, stream));
    } else {
        hipLaunchKernelGGL(k_publish_count, dim3(1), dim3(WAVE), 0, stream, s.hdr, 0, n_out_dev);
        SPC_LAUNCHED("k_publish_count");
    }
    if (!strided_count_only) {
        // Everything after the count is sized by the caller's capacity and reads
        // M on the device (a count above the capacity reads as 0), so nothing
        // after this point waits for the host.
        const int64_t cap = std::min<int64_t>(out_cap, p.m_max);
        hipLaunchKernelGGL(k_bitmap_emit, dim3(unsigned(p.bm_blocks)), dim3(KB), 0, stream, bitmap, p.nwords, bsums,
                           int32_t(scanned), prefix, reinterpret_cast<int4*>(out_coords), int64_t(out_cap), s.hdr, p.g);
        SPC_LAUNCHED("k_bitmap_emit");
        // Everything goes on the caller's stream: side streams inside the call
        // overlapped the two sides' sorts on the GPU, but their fork and join
        // events cost more host time than they saved; a caller overlaps whole
        // maps with its other work instead.
        if (p.K <= ROWPASS_KMAX) {
            // the input side (nbr_in, its masks and its order), then the output
            // side, whose rows gather their entries through the input table,
            // with their masks and counts
            if (nbr_in && n > 0) {
                hipLaunchKernelGGL(k_in_rows, dim3(unsigned(nblk)), dim3(KB), 0, stream, c4, n, int64_t(out_cap),
                                   p.g, bitmap, prefix, nbr_in, order_in ? s.mask[1] : nullptr, s.hdr);
                SPC_LAUNCHED("k_in_rows");
            }
            auto rows_kernel = p.g.dense ? k_out_rows<TBL_GRID, false>
                                         : p.g.occ ? k_out_rows<TBL_FILTERED, false> : k_out_rows<TBL_HASH, false>;
            hipLaunchKernelGGL(rows_kernel, dim3(unsigned(std::max<int64_t>(ceil_div(cap, KB), 1))), dim3(KB), 0, stream,
                               reinterpret_cast<const int4*>(out_coords), -1, int64_t(out_cap), p.g, table, mask, occ,
                               nbr, (pairs || order) ? s.mask[0] : nullptr, pairs ? s.counts : nullptr, s.hdr,
                               coord_err);
            SPC_LAUNCHED("k_out_rows");
            // both orders from the row kernels' masks, sharing each pass's launches
            OrderJob jobs[2];
            int nj = 0;
            if (order_in && n > 0) jobs[nj++] = OrderJob{nbr_in, n, n, n, true, 1, order_in};
            if (order) jobs[nj++] = OrderJob{nbr, -1, cap, int64_t(out_cap), true, 0, order};
            if ((st = sort_orders(p, s, jobs, nj, stream)) != SPC_OK) return st;
        } else {
            // larger kernels: the output-side map is the transpose of the
            // input-side one, scattered into a map filled with -1
            hipLaunchKernelGGL(k_fill_map, dim3(grid_for(cap * p.K, KB, 4096)), dim3(KB), 0, stream, nbr, p.K,
                               int64_t(out_cap), s.hdr);
            SPC_LAUNCHED("k_fill_map");
            hipLaunchKernelGGL(k_strided_maps, dim3(unsigned(std::max<int64_t>(ceil_div(entries, KB), 1))), dim3(KB),
                               0, stream, c4, n, int64_t(out_cap), p.g, bitmap, prefix, nbr, nbr_in, s.hdr, coord_err);
            SPC_LAUNCHED("k_strided_maps");
            // the input-side order (its own row pass and sort)
            if (order_in) {
                st = sort_rows(p, nbr_in, n, n, n, s, false, 1, order_in, stream);
                if (st != SPC_OK) return st;
            }
            if (pairs || order) {
                st = row_pass(p, nbr, -1, cap, int64_t(out_cap), s, s.mask[0], pairs ? s.counts : nullptr, stream);
                if (st != SPC_OK) return st;
            }
        }
        if (order && p.K > ROWPASS_KMAX) {
            st = sort_rows(p, nbr, -1, cap, int64_t(out_cap), s, true, 0, order, stream);
            if (st != SPC_OK) return st;
        }
        if (pairs) {
            st = map_pairs(p, nbr, -1, cap, int64_t(out_cap), s, pair_ptr, pair_in, pair_out, stream);
            if (st != SPC_OK) return st;
        }
    }
    if (!wait) return SPC_OK;  // flags reach coord_err through the row kernels; the count is on the device
    SPC_HIP(hipEventSynchronize(hc->ev));
    const uint32_t host_hdr[2] = {hc->words[H_FLAGS], hc->words[H_NOUT]};
    const int64_t M = host_hdr[H_NOUT];
    *n_out = M;
    if (host_hdr[H_FLAGS] & (SPC_COORD_OUT_OF_RANGE | SPC_COORD_DUPLICATE))
        return fail(SPC_ERR_COORD, "input coordinates: %s%s",
                    (host_hdr[H_FLAGS] & SPC_COORD_OUT_OF_RANGE) ? "out of range " : "",
                    (host_hdr[H_FLAGS] & SPC_COORD_DUPLICATE) ? "duplicate" : "");
    if (!strided_count_only && M > out_cap)
        return fail(SPC_ERR_CAPACITY, "%lld output sites exceed out_cap=%lld", (long long)M, (long long)out_cap);
    return SPC_OK;
}

}  // namespace
}  // namespace spc

extern "C" spc_status spc_build_kmap(const spc_geom* g, const int32_t* coords, int64_t n_in, int32_t* out_coords,
                                     int64_t out_cap, int64_t* n_out, int32_t* nbr, int32_t* nbr_in,
                                     int32_t* pair_ptr, int32_t* pair_in, int32_t* pair_out, int64_t pair_cap,
                                     int32_t* order, int32_t* order_in, int32_t* coord_err, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
    clear_error();
    return build_kmap(g, coords, n_in, out_coords, out_cap, n_out, nullptr, nbr, nbr_in, pair_ptr, pair_in, pair_out,
                      pair_cap, order, order_in, coord_err, ws, ws_bytes, stream);
}

extern "C" spc_status spc_build_kmap_async(const spc_geom* g, const int32_t* coords, int64_t n_in,
                                           int32_t* out_coords, int64_t out_cap, int32_t* n_out_dev, int32_t* nbr,
                                           int32_t* nbr_in, int32_t* pair_ptr, int32_t* pair_in, int32_t* pair_out,
                                           int64_t pair_cap, int32_t* order, int32_t* order_in, int32_t* coord_err,
                                           void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    if (!n_out_dev) return fail(SPC_ERR_ARG, "n_out_dev is NULL");
    return build_kmap(g, coords, n_in, out_coords, out_cap, nullptr, n_out_dev, nbr, nbr_in, pair_ptr, pair_in,
                      pair_out, pair_cap, order, order_in, coord_err, ws, ws_bytes, stream);
}
