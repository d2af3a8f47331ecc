// Kernel-map construction on the GPU: hash build, per-offset probes, strided
// output sites and CSR pair lists.
//
// Hash table: open addressing with linear probing over 64-bit slots that pack
// (key << 32) | row, so one 8-byte load answers a probe and one 64-bit CAS
// claims a slot (the single-slot table of spconv's hash.HashTable on the
// context7 spconv page).  Keys are ((b*Z + z)*Y + y)*X + x, the packing of the
// MLX sparse/conv.py page's build_indice_map, bounded below 2^32 so the
// all-ones slot can mark "empty".  Capacity is a power of two >= 2N.
//
// Strided output sites are marked in a bitmap over the output grid; a
// per-word exclusive prefix of popcounts then gives, for any output site, its
// row in (b, z, y, x) order (rank = prefix[word] + popcount of the lower bits),
// so sorted output coordinates need no sort and no second table.
//
// Pair lists are compacted in (offset, output row) order with a per-block
// count pass, one exclusive scan, and an ordered ballot/prefix write pass.
#include <stdio.h>

#include <algorithm>

#include "common.h"

namespace spc {
namespace {

constexpr uint64_t EMPTY_SLOT = ~0ull;
constexpr int KB = 256;          // threads (= rows) per block of the per-row kernels
constexpr int MAX_K = 343;       // up to 7 x 7 x 7 offsets
constexpr int WORDS_PER_THREAD = 8;
constexpr int SCAN_THREADS = 1024;

struct KGeom {
    int32_t batch, Z, Y, X;      // input grid
    int32_t kz, ky, kx;
    int32_t sz, sy, sx;
    int32_t pz, py, px;
    int32_t dz, dy, dx;
    int32_t oz, oy, ox;          // output grid (equal to the input grid for subm)
};

// Header at the start of the workspace.
enum { H_FLAGS = 0, H_NOUT = 1, H_WORDS = 64 };

__device__ __forceinline__ uint32_t mix32(uint32_t k) {
    // murmur3's 32-bit finaliser
    k ^= k >> 16;
    k *= 0x85ebca6bu;
    k ^= k >> 13;
    k *= 0xc2b2ae35u;
    k ^= k >> 16;
    return k;
}

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
    uint32_t h = mix32(key) & mask;
    // at most N of the >= 2N slots are ever taken, so an empty slot is always found
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
    uint32_t h = mix32(key) & mask;
    for (uint32_t step = 0; step <= mask; ++step) {
        const uint64_t v = table[h];
        if (v == EMPTY_SLOT) return -1;
        if (uint32_t(v >> 32) == key) return int32_t(uint32_t(v));
        h = (h + 1) & mask;
    }
    return -1;
}

// Adds this wave's hit count for offset k to the block's LDS counter.
__device__ __forceinline__ void count_hits(bool hit, int32_t* cnt, int k) {
    const uint64_t b = __ballot(hit);
    if ((threadIdx.x & (WAVE - 1)) == 0 && b) atomicAdd(cnt + k, __popcll(b));
}

// ---------------------------------------------------------------- kernels

// Fills the table with the empty marker, zeroes the bitmap and the header.
__global__ void k_clear(uint64_t* __restrict__ table, int64_t cap, uint32_t* __restrict__ bitmap,
                        int64_t nwords, uint32_t* __restrict__ hdr) {
    const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    if (t < H_WORDS) hdr[t] = 0u;
    u32x4 ones = {~0u, ~0u, ~0u, ~0u};
    for (int64_t i = t; i < cap / 2; i += stride) st16(table + 2 * i, ones);
    for (int64_t i = t; i < nwords / 4; i += stride) st16(bitmap + 4 * i, zero4());
}

// Inserts every in-range input row; flags bad and duplicate rows.  For a
// strided geometry it also sets the bitmap bit of every output site the row
// reaches: o = (c + pad - k*dil) / stride per axis, exact and inside the grid.
template <bool STRIDED>
__global__ __launch_bounds__(KB) void k_insert(const int4* __restrict__ coords, int32_t n, KGeom g,
                                               uint64_t* table, uint32_t mask,
                                               uint32_t* bitmap, uint32_t* hdr) {
    const int32_t i = blockIdx.x * KB + threadIdx.x;
    if (i >= n) return;
    const int4 c = coords[i];
    if (!in_grid(c, g)) {
        atomicOr(hdr + H_FLAGS, SPC_COORD_OUT_OF_RANGE);
        return;
    }
    table_insert(table, mask, in_key(c.x, c.y, c.z, c.w, g), uint32_t(i), hdr + H_FLAGS);
    if (!STRIDED) return;
    int oz[8], oy[8], ox[8];
    int nz = 0, ny = 0, nx = 0;
    for (int k = 0; k < g.kz; ++k) {
        const int num = c.y + g.pz - k * g.dz;
        if (num >= 0 && num % g.sz == 0 && num / g.sz < g.oz && nz < 8) oz[nz++] = num / g.sz;
    }
    for (int k = 0; k < g.ky; ++k) {
        const int num = c.z + g.py - k * g.dy;
        if (num >= 0 && num % g.sy == 0 && num / g.sy < g.oy && ny < 8) oy[ny++] = num / g.sy;
    }
    for (int k = 0; k < g.kx; ++k) {
        const int num = c.w + g.px - k * g.dx;
        if (num >= 0 && num % g.sx == 0 && num / g.sx < g.ox && nx < 8) ox[nx++] = num / g.sx;
    }
    for (int a = 0; a < nz; ++a)
        for (int b = 0; b < ny; ++b)
            for (int d = 0; d < nx; ++d) {
                const uint32_t key = out_key(c.x, oz[a], oy[b], ox[d], g);
                atomicOr(bitmap + (key >> 5), 1u << (key & 31u));
            }
}

// Submanifold probes: nbr[k*n + i] = row at coords[i] + d_k, else -1, with
// d_k = (kz - KZ/2, ky - KY/2, kx - KX/2), z slowest.  Optionally counts the
// hits of each offset in this block into counts[k*nblk + block].
__global__ __launch_bounds__(KB) void k_subm_probe(const int4* __restrict__ coords, int32_t n, KGeom g,
                                                   const uint64_t* __restrict__ table, uint32_t mask,
                                                   int32_t* __restrict__ nbr, int32_t* __restrict__ counts,
                                                   const uint32_t* hdr, int32_t* coord_err) {
    __shared__ int32_t cnt[MAX_K];
    const int K = g.kz * g.ky * g.kx;
    for (int k = threadIdx.x; k < K; k += KB) cnt[k] = 0;
    if (coord_err && blockIdx.x == 0 && threadIdx.x == 0) *coord_err = int32_t(hdr[H_FLAGS]);
    __syncthreads();
    const int32_t i = blockIdx.x * KB + threadIdx.x;
    const bool live = i < n;
    int4 c = make_int4(-1, -1, -1, -1);
    if (live) c = coords[i];
    const bool ok = live && in_grid(c, g);
    const int rz = g.kz / 2, ry = g.ky / 2, rx = g.kx / 2;
    int k = 0;
    for (int a = 0; a < g.kz; ++a) {
        const int z = c.y + a - rz;
        for (int b = 0; b < g.ky; ++b) {
            const int y = c.z + b - ry;
            for (int d = 0; d < g.kx; ++d, ++k) {
                const int x = c.w + d - rx;
                int32_t v = -1;
                if (ok && (unsigned)z < (unsigned)g.Z && (unsigned)y < (unsigned)g.Y &&
                    (unsigned)x < (unsigned)g.X)
                    v = table_find(table, mask, in_key(c.x, z, y, x, g));
                if (live) nbr[int64_t(k) * n + i] = v;
                if (counts) count_hits(v >= 0, cnt, k);
            }
        }
    }
    if (!counts) return;
    __syncthreads();
    for (int kk = threadIdx.x; kk < K; kk += KB) counts[int64_t(kk) * gridDim.x + blockIdx.x] = cnt[kk];
}

// Popcount of each thread's WORDS_PER_THREAD bitmap words, summed per block.
__global__ __launch_bounds__(KB) void k_bitmap_count(const uint32_t* __restrict__ bitmap, int64_t nwords,
                                                     int32_t* __restrict__ block_sums) {
    __shared__ int32_t red[KB / WAVE];
    const int64_t w0 = (int64_t(blockIdx.x) * KB + threadIdx.x) * WORDS_PER_THREAD;
    int s = 0;
    if (w0 < nwords) {
        const u32x4 a = ld16(bitmap + w0), b = ld16(bitmap + w0 + 4);
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
    }
}

// Block-wide exclusive scan of one int per thread; returns the block total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_waves, int& total) {
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    int incl = v;
    for (int off = 1; off < WAVE; off <<= 1) {
        const int u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
    }
    if (lane == WAVE - 1) lds_waves[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < NT / WAVE; ++w) {
        const int s = lds_waves[w];
        if (w < wave) before += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// One-workgroup exclusive scan of data[0, L) in place (L < 2^31 total).
// With ptr != NULL, ptr[k] = data[k * nblk] (after the scan) for k < K and
// ptr[K] = total: the CSR offsets of the (offset, block) count matrix.
// With total_out != NULL the total is also stored there.
__global__ __launch_bounds__(SCAN_THREADS) void k_scan(int32_t* __restrict__ data, int64_t L, int32_t* ptr,
                                                       int K, int64_t nblk, uint32_t* total_out) {
    __shared__ int waves[SCAN_THREADS / WAVE];
    const int64_t per = (L + SCAN_THREADS - 1) / SCAN_THREADS;
    const int64_t lo = min<int64_t>(L, per * threadIdx.x), hi = min<int64_t>(L, lo + per);
    int s = 0;
    for (int64_t j = lo; j < hi; ++j) s += data[j];
    int total;
    int run = block_exclusive_scan<SCAN_THREADS>(s, waves, total);
    for (int64_t j = lo; j < hi; ++j) {
        const int v = data[j];
        data[j] = run;
        run += v;
    }
    __syncthreads();
    if (ptr) {
        for (int k = threadIdx.x; k < K; k += SCAN_THREADS) ptr[k] = nblk > 0 ? data[int64_t(k) * nblk] : 0;
        if (threadIdx.x == 0) ptr[K] = total;
    }
    if (total_out && threadIdx.x == 0) *total_out = uint32_t(total);
}

// Writes each word's exclusive rank prefix and the output coordinates of
// its set bits, in (b, z, y, x) order.
__global__ __launch_bounds__(KB) void k_bitmap_emit(const uint32_t* __restrict__ bitmap, int64_t nwords,
                                                    const int32_t* __restrict__ block_offs,
                                                    uint32_t* __restrict__ prefix, int4* __restrict__ out_coords,
                                                    KGeom g) {
    __shared__ int waves[KB / WAVE];
    const int64_t w0 = (int64_t(blockIdx.x) * KB + threadIdx.x) * WORDS_PER_THREAD;
    uint32_t w[WORDS_PER_THREAD] = {0, 0, 0, 0, 0, 0, 0, 0};
    int s = 0;
    if (w0 < nwords) {
        const u32x4 a = ld16(bitmap + w0), b = ld16(bitmap + w0 + 4);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        for (int j = 0; j < WORDS_PER_THREAD; ++j) s += __popc(w[j]);
    }
    int total;
    int run = block_offs[blockIdx.x] + block_exclusive_scan<KB>(s, waves, total);
    if (w0 >= nwords) return;
    const int64_t plane = int64_t(g.oy) * g.ox, vol = plane * g.oz;
    for (int j = 0; j < WORDS_PER_THREAD; ++j) {
        prefix[w0 + j] = uint32_t(run);
        uint32_t bits = w[j];
        while (bits) {
            const int bit = __ffs(bits) - 1;
            bits &= bits - 1;
            const int64_t key = (w0 + j) * 32 + bit;
            const int b = int(key / vol);
            const int64_t r = key - int64_t(b) * vol;
            const int z = int(r / plane);
            const int64_t r2 = r - int64_t(z) * plane;
            out_coords[run++] = make_int4(b, z, int(r2 / g.ox), int(r2 % g.ox));
        }
    }
}

// Strided maps.  Blocks [0, mblk) handle output rows: nbr[k*M + o] = input
// row at o*stride - pad + k*dil, else -1 (and per-block hit counts).  Blocks
// [mblk, ...) handle input rows: nbr_in[k*n + i] = rank of the output site
// that input i reaches through offset k, else -1.
__global__ __launch_bounds__(KB) void k_strided_maps(const int4* __restrict__ coords, int32_t n,
                                                     const int4* __restrict__ out_coords, int32_t M,
                                                     int32_t mblk, KGeom g,
                                                     const uint64_t* __restrict__ table, uint32_t mask,
                                                     const uint32_t* __restrict__ bitmap,
                                                     const uint32_t* __restrict__ prefix,
                                                     int32_t* __restrict__ nbr, int32_t* __restrict__ nbr_in,
                                                     int32_t* __restrict__ counts, const uint32_t* hdr,
                                                     int32_t* coord_err) {
    __shared__ int32_t cnt[MAX_K];
    const int K = g.kz * g.ky * g.kx;
    if (coord_err && blockIdx.x == 0 && threadIdx.x == 0) *coord_err = int32_t(hdr[H_FLAGS]);
    if (int32_t(blockIdx.x) < mblk) {
        for (int k = threadIdx.x; k < K; k += KB) cnt[k] = 0;
        __syncthreads();
        const int32_t o = blockIdx.x * KB + threadIdx.x;
        const bool live = o < M;
        int4 c = make_int4(0, 0, 0, 0);
        if (live) c = out_coords[o];
        int k = 0;
        for (int a = 0; a < g.kz; ++a) {
            const int z = c.y * g.sz - g.pz + a * g.dz;
            for (int b = 0; b < g.ky; ++b) {
                const int y = c.z * g.sy - g.py + b * g.dy;
                for (int d = 0; d < g.kx; ++d, ++k) {
                    const int x = c.w * g.sx - g.px + d * g.dx;
                    int32_t v = -1;
                    if (live && (unsigned)z < (unsigned)g.Z && (unsigned)y < (unsigned)g.Y &&
                        (unsigned)x < (unsigned)g.X)
                        v = table_find(table, mask, in_key(c.x, z, y, x, g));
                    if (live) nbr[int64_t(k) * M + o] = v;
                    if (counts) count_hits(v >= 0, cnt, k);
                }
            }
        }
        if (!counts) return;
        __syncthreads();
        for (int kk = threadIdx.x; kk < K; kk += KB) counts[int64_t(kk) * mblk + blockIdx.x] = cnt[kk];
        return;
    }
    const int32_t i = (blockIdx.x - mblk) * KB + threadIdx.x;
    if (i >= n) return;
    const int4 c = coords[i];
    const bool ok = in_grid(c, g);
    int k = 0;
    for (int a = 0; a < g.kz; ++a) {
        const int nz = c.y + g.pz - a * g.dz;
        const bool vz = nz >= 0 && nz % g.sz == 0 && nz / g.sz < g.oz;
        for (int b = 0; b < g.ky; ++b) {
            const int ny = c.z + g.py - b * g.dy;
            const bool vy = ny >= 0 && ny % g.sy == 0 && ny / g.sy < g.oy;
            for (int d = 0; d < g.kx; ++d, ++k) {
                const int nx = c.w + g.px - d * g.dx;
                const bool vx = nx >= 0 && nx % g.sx == 0 && nx / g.sx < g.ox;
                int32_t v = -1;
                if (ok && vz && vy && vx) {
                    const uint32_t key = out_key(c.x, nz / g.sz, ny / g.sy, nx / g.sx, g);
                    const uint32_t word = key >> 5, bit = key & 31u;
                    v = int32_t(prefix[word] + __popc(bitmap[word] & ((1u << bit) - 1u)));
                }
                nbr_in[int64_t(k) * n + i] = v;
            }
        }
    }
}

// Ordered compaction of one (block of rows, offset) tile of the map into the
// CSR pair lists at the scanned offset offs[k*nblk + block].
__global__ __launch_bounds__(KB) void k_compact_pairs(const int32_t* __restrict__ nbr, int32_t rows,
                                                      const int32_t* __restrict__ offs,
                                                      int32_t* __restrict__ pair_in,
                                                      int32_t* __restrict__ pair_out) {
    __shared__ int waves[KB / WAVE];
    const int k = blockIdx.y;
    const int32_t o = blockIdx.x * KB + threadIdx.x;
    int32_t v = -1;
    if (o < rows) v = nbr[int64_t(k) * rows + o];
    int total;
    const int pos = block_exclusive_scan<KB>(v >= 0 ? 1 : 0, waves, total);
    if (v >= 0) {
        const int64_t at = int64_t(offs[int64_t(k) * gridDim.x + blockIdx.x]) + pos;
        pair_in[at] = v;
        pair_out[at] = o;
    }
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
    int64_t m_max;               // upper bound of the output row count
    int64_t cblk;                // count-matrix blocks per offset (max over phases)
    int64_t bm_blocks;           // bitmap count/emit blocks
    // workspace offsets
    size_t off_table, off_counts, off_bitmap, off_prefix, off_bsums, total;
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
        if (!g.subm) {
            if (g.stride[a] <= 0 || g.dil[a] <= 0 || g.pad[a] < 0)
                return fail(SPC_ERR_ARG, "axis %d: stride=%d dil=%d pad=%d invalid", a, g.stride[a], g.dil[a], g.pad[a]);
        }
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
    const uint64_t in_vol = uint64_t(g.batch) * k.Z * k.Y * k.X;
    if (in_vol >= (uint64_t(1) << 32))
        return fail(SPC_ERR_UNSUPPORTED, "batch*Z*Y*X = %llu must be below 2^32", (unsigned long long)in_vol);
    p.out_vol = g.subm ? 0 : int64_t(uint64_t(g.batch) * k.oz * k.oy * k.ox);
    if (uint64_t(p.out_vol) >= (uint64_t(1) << 32))
        return fail(SPC_ERR_UNSUPPORTED, "output grid volume %lld must be below 2^32", (long long)p.out_vol);
    if (int64_t(p.K) * n_in >= (int64_t(1) << 31))
        return fail(SPC_ERR_UNSUPPORTED, "K*n_in=%lld must be below 2^31", (long long)(int64_t(p.K) * n_in));
    p.n = n_in;
    p.cap_log2 = 6;
    while ((int64_t(1) << p.cap_log2) < 2 * n_in) ++p.cap_log2;
    p.cap = int64_t(1) << p.cap_log2;
    const int64_t wpb = int64_t(KB) * WORDS_PER_THREAD;
    p.nwords = g.subm ? 0 : ceil_div(ceil_div(p.out_vol, 32), wpb) * wpb;
    p.bm_blocks = p.nwords / wpb;
    p.m_max = g.subm ? n_in : std::min<int64_t>(int64_t(p.K) * n_in, p.out_vol);
    p.cblk = std::max<int64_t>(ceil_div(n_in, KB), ceil_div(p.m_max, KB));
    size_t off = 256;
    p.off_table = off;   off = align_up(off + size_t(p.cap) * 8, 256);
    p.off_counts = off;  off = align_up(off + size_t(p.K) * p.cblk * 4, 256);
    p.off_bitmap = off;  off = align_up(off + size_t(p.nwords) * 4, 256);
    p.off_prefix = off;  off = align_up(off + size_t(p.nwords) * 4, 256);
    p.off_bsums = off;   off = align_up(off + size_t(p.bm_blocks) * 4 + 4, 256);
    p.total = off;
    return SPC_OK;
}

inline unsigned grid_for(int64_t work, int64_t per_block, int64_t cap = 1 << 16) {
    int64_t b = ceil_div(std::max<int64_t>(work, 1), per_block);
    return unsigned(std::min<int64_t>(std::max<int64_t>(b, 1), cap));
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

extern "C" spc_status spc_build_kmap(const spc_geom* gp, const int32_t* coords, int64_t n_in,
                                     int32_t* out_coords, int64_t out_cap, int64_t* n_out,
                                     int32_t* nbr, int32_t* nbr_in,
                                     int32_t* pair_ptr, int32_t* pair_in, int32_t* pair_out, int64_t pair_cap,
                                     int32_t* coord_err, void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    Plan p;
    spc_status st = make_plan(gp, n_in, p);
    if (st != SPC_OK) return st;
    const bool subm = gp->subm != 0;
    const bool strided_count_only = !subm && out_coords == nullptr;
    if (!n_out) return fail(SPC_ERR_ARG, "n_out is NULL");
    if (n_in > 0 && !coords) return fail(SPC_ERR_ARG, "coords is NULL");
    if (!ws) return fail(SPC_ERR_ARG, "workspace is NULL");
    if (ws_bytes < p.total) return fail(SPC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, p.total);
    const bool pairs = pair_ptr || pair_in || pair_out;
    if (pairs && !(pair_ptr && pair_in && pair_out)) return fail(SPC_ERR_ARG, "pair_ptr/pair_in/pair_out must be all set or all NULL");
    if (pairs && pair_cap < int64_t(p.K) * n_in) return fail(SPC_ERR_ARG, "pair_cap=%lld < K*n_in=%lld", (long long)pair_cap, (long long)(int64_t(p.K) * n_in));
    if (!strided_count_only && !nbr) return fail(SPC_ERR_ARG, "nbr is NULL");
    if (!subm && !strided_count_only && out_cap < 0) return fail(SPC_ERR_ARG, "out_cap < 0");
    const void* ptrs[] = {coords, out_coords, nbr, nbr_in, pair_ptr, pair_in, pair_out, coord_err, ws};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");

    char* base = static_cast<char*>(ws);
    uint32_t* hdr = reinterpret_cast<uint32_t*>(base);
    uint64_t* table = reinterpret_cast<uint64_t*>(base + p.off_table);
    int32_t* counts = reinterpret_cast<int32_t*>(base + p.off_counts);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + p.off_bitmap);
    uint32_t* prefix = reinterpret_cast<uint32_t*>(base + p.off_prefix);
    int32_t* bsums = reinterpret_cast<int32_t*>(base + p.off_bsums);
    const int4* c4 = reinterpret_cast<const int4*>(coords);
    const int32_t n = int32_t(n_in);
    const uint32_t mask = uint32_t(p.cap - 1);
    const unsigned nblk = unsigned(std::max<int64_t>(ceil_div(n, KB), 1));

    hipLaunchKernelGGL(k_clear, dim3(grid_for(std::max(p.cap / 2, p.nwords / 4), KB, 4096)), dim3(KB), 0, stream,
                       table, p.cap, bitmap, p.nwords, hdr);
    SPC_LAUNCHED("k_clear");

    if (subm) {
        if (n > 0) {
            hipLaunchKernelGGL(k_insert<false>, dim3(nblk), dim3(KB), 0, stream, c4, n, p.g, table, mask,
                               bitmap, hdr);
            SPC_LAUNCHED("k_insert");
        }
        hipLaunchKernelGGL(k_subm_probe, dim3(nblk), dim3(KB), 0, stream, c4, n, p.g, table, mask, nbr,
                           pairs ? counts : nullptr, hdr, coord_err);
        SPC_LAUNCHED("k_subm_probe");
        if (pairs) {
            const int64_t cb = n > 0 ? int64_t(nblk) : 0;
            hipLaunchKernelGGL(k_scan, dim3(1), dim3(SCAN_THREADS), 0, stream, counts, int64_t(p.K) * cb,
                               pair_ptr, p.K, cb, (uint32_t*)nullptr);
            SPC_LAUNCHED("k_scan");
            if (n > 0) {
                hipLaunchKernelGGL(k_compact_pairs, dim3(nblk, p.K), dim3(KB), 0, stream, nbr, n, counts,
                                   pair_in, pair_out);
                SPC_LAUNCHED("k_compact_pairs");
            }
        }
        *n_out = n_in;
        return SPC_OK;
    }

    // strided: output sites into the bitmap, then count them
    if (n > 0) {
        hipLaunchKernelGGL(k_insert<true>, dim3(nblk), dim3(KB), 0, stream, c4, n, p.g, table, mask, bitmap, hdr);
        SPC_LAUNCHED("k_insert");
    }
    if (p.bm_blocks > 0) {
        hipLaunchKernelGGL(k_bitmap_count, dim3(unsigned(p.bm_blocks)), dim3(KB), 0, stream, bitmap, p.nwords, bsums);
        SPC_LAUNCHED("k_bitmap_count");
    }
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(SCAN_THREADS), 0, stream, bsums, p.bm_blocks, (int32_t*)nullptr, 0,
                       int64_t(0), hdr + H_NOUT);
    SPC_LAUNCHED("k_scan");
    uint32_t host_hdr[2] = {0, 0};
    SPC_HIP(hipMemcpyAsync(host_hdr, hdr, sizeof(host_hdr), hipMemcpyDeviceToHost, stream));
    SPC_HIP(hipStreamSynchronize(stream));
    const int64_t M = host_hdr[H_NOUT];
    *n_out = M;
    if (host_hdr[H_FLAGS]) {
        if (coord_err) SPC_HIP(hipMemcpyAsync(coord_err, hdr, 4, hipMemcpyDeviceToDevice, stream));
        return fail(SPC_ERR_COORD, "input coordinates: %s%s",
                    (host_hdr[H_FLAGS] & SPC_COORD_OUT_OF_RANGE) ? "out of range " : "",
                    (host_hdr[H_FLAGS] & SPC_COORD_DUPLICATE) ? "duplicate" : "");
    }
    if (strided_count_only) return SPC_OK;
    if (M > out_cap) return fail(SPC_ERR_CAPACITY, "%lld output sites exceed out_cap=%lld", (long long)M, (long long)out_cap);

    if (p.bm_blocks > 0) {
        hipLaunchKernelGGL(k_bitmap_emit, dim3(unsigned(p.bm_blocks)), dim3(KB), 0, stream, bitmap, p.nwords, bsums,
                           prefix, reinterpret_cast<int4*>(out_coords), p.g);
        SPC_LAUNCHED("k_bitmap_emit");
    }
    const int32_t mblk = int32_t(ceil_div(M, KB));
    const int32_t iblk = nbr_in ? int32_t(ceil_div(n, KB)) : 0;
    hipLaunchKernelGGL(k_strided_maps, dim3(unsigned(std::max(mblk + iblk, 1))), dim3(KB), 0, stream, c4, n,
                       reinterpret_cast<const int4*>(out_coords), int32_t(M), mblk, p.g, table, mask, bitmap, prefix,
                       nbr, nbr_in, pairs ? counts : nullptr, hdr, coord_err);
    SPC_LAUNCHED("k_strided_maps");
    if (pairs) {
        hipLaunchKernelGGL(k_scan, dim3(1), dim3(SCAN_THREADS), 0, stream, counts, int64_t(p.K) * mblk, pair_ptr,
                           p.K, int64_t(mblk), (uint32_t*)nullptr);
        SPC_LAUNCHED("k_scan");
        if (mblk > 0) {
            hipLaunchKernelGGL(k_compact_pairs, dim3(unsigned(mblk), p.K), dim3(KB), 0, stream, nbr, int32_t(M), counts,
                               pair_in, pair_out);
            SPC_LAUNCHED("k_compact_pairs");
        }
    }
    return SPC_OK;
}
