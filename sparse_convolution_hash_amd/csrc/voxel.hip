// Point-cloud voxelisation on the GPU (spconv's PointToVoxel, USAGE.md:
// "spconv.pytorch.utils API Reference" and the PointToVoxel example), and the
// per-point gather of voxel features by voxel id.
//
// Points fall into voxels of a grid over a box; the voxels are numbered in
// order of their first point, each keeps its first max_points points in
// point order, and once max_voxels voxels exist further voxels are dropped.
// Every step below is deterministic (no result depends on atomics' order):
//
//   1. clear     the hash table (64-bit slots, all ones = empty) and counters
//   2. insert    voxel key of each point (fp32 floor((p - min) / vsize)); a
//                slot holds (key << 32 | smallest point index): claimed with
//                a CAS, then lowered with a 64-bit atomicMin, which keeps the
//                key half and the smaller index
//   3. first     a point is its voxel's first iff the slot's index is its own;
//                per-block counts of first points
//   4. scan      exclusive scan of the block counts (total = voxels found)
//   5. number    each first point numbers its voxel (block offset + rank)
//   6. keys      each point takes its voxel's number as sort key (dropped and
//                outside points sort last)
//   7. sort      stable LSD radix passes (radix.h): points grouped by voxel,
//                in point order inside each voxel
//   8. segments  each voxel's run [start, end) in the sorted order
//   9. write     one thread per (voxel, point slot): the point, or the mean of
//                the voxel's points (empty_mean) or zeros; counts, ZYX
//                coordinates and the point -> voxel ids
#include <math.h>

#include "common.h"
#include "radix.h"

namespace spc {
namespace {

constexpr int VT = 256;                // threads per block of the per-point kernels
constexpr int VSCAN = 1024;            // threads of the one-block scan
constexpr uint64_t EMPTY = ~0ull;
constexpr uint32_t NO_KEY = ~0u;
constexpr int MAX_FEATURES = 64;
enum { V_TOTAL = 0, V_WORDS = 64 };    // header words

struct VoxGeom {
    float lo[3], vs[3];                // box minimum and voxel size (x, y, z)
    int32_t ext[3];                    // voxels per axis (x, y, z)
};

__device__ __forceinline__ uint32_t mix32(uint32_t k) {
    // murmur3's 32-bit finaliser
    k ^= k >> 16;
    k *= 0x85ebca6bu;
    k ^= k >> 13;
    k *= 0xc2b2ae35u;
    k ^= k >> 16;
    return k;
}

__global__ void k_vox_clear(uint64_t* __restrict__ table, int64_t cap, uint32_t* __restrict__ hdr,
                            int32_t* __restrict__ zero, int64_t nzero) {
    const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    if (t < V_WORDS) hdr[t] = 0u;
    const u32x4 ones = {~0u, ~0u, ~0u, ~0u};
    for (int64_t i = t; i < cap / 2; i += stride) st16(table + 2 * i, ones);
    for (int64_t i = t; i < nzero; i += stride) zero[i] = 0;
}

__global__ __launch_bounds__(VT) void k_vox_insert(const float* __restrict__ pts, int32_t n, int32_t F, VoxGeom g,
                                                   uint64_t* __restrict__ table, uint32_t mask,
                                                   uint32_t* __restrict__ keyv, int32_t* __restrict__ slot) {
    const int i = int(blockIdx.x) * VT + int(threadIdx.x);
    if (i >= n) return;
    const float* p = pts + int64_t(i) * F;
    int c[3];
    bool inside = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const float f = floorf(__fdiv_rn(p[a] - g.lo[a], g.vs[a]));  // each operation rounded to nearest
        inside = inside && f >= 0.f && f < float(g.ext[a]);         // (false for NaN)
        c[a] = inside ? int(f) : 0;
    }
    if (!inside) {
        keyv[i] = NO_KEY;
        slot[i] = -1;
        return;
    }
    const uint32_t key = uint32_t((uint64_t(c[2]) * uint64_t(g.ext[1]) + uint64_t(c[1])) * uint64_t(g.ext[0]) + c[0]);
    const unsigned long long v = (static_cast<unsigned long long>(key) << 32) | uint32_t(i);
    uint32_t h = mix32(key) & mask;
    int32_t s = -1;
    // at most n of the >= 2n slots are ever taken, so an empty slot is always found
    for (uint32_t step = 0; step <= mask; ++step) {
        const unsigned long long prev = atomicCAS(reinterpret_cast<unsigned long long*>(table + h), EMPTY, v);
        if (prev == EMPTY) {
            s = int32_t(h);
            break;
        }
        if (uint32_t(prev >> 32) == key) {
            atomicMin(reinterpret_cast<unsigned long long*>(table + h), v);  // same key half: keeps the smaller index
            s = int32_t(h);
            break;
        }
        h = (h + 1) & mask;
    }
    keyv[i] = key;
    slot[i] = s;
}

__device__ __forceinline__ bool is_first(const uint64_t* __restrict__ table, const int32_t* __restrict__ slot,
                                         int i, int n) {
    if (i >= n) return false;
    const int32_t s = slot[i];
    return s >= 0 && uint32_t(table[s]) == uint32_t(i);
}

__global__ __launch_bounds__(VT) void k_vox_first(const uint64_t* __restrict__ table, const int32_t* __restrict__ slot,
                                                  int32_t n, int32_t* __restrict__ btot) {
    __shared__ int waves[VT / WAVE];
    const int i = int(blockIdx.x) * VT + int(threadIdx.x);
    int total;
    block_exclusive_scan<VT>(is_first(table, slot, i, n) ? 1 : 0, waves, total);
    if (threadIdx.x == 0) btot[blockIdx.x] = total;
}

// One block: exclusive scan of btot[0, nb) into boff; the total into hdr.
__global__ __launch_bounds__(VSCAN) void k_vox_scan(const int32_t* __restrict__ btot, int32_t nb,
                                                    int32_t* __restrict__ boff, uint32_t* __restrict__ hdr) {
    __shared__ int waves[VSCAN / WAVE];
    const int per = (nb + VSCAN - 1) / VSCAN;
    const int b0 = int(threadIdx.x) * per;
    int s = 0;
    for (int j = 0; j < per; ++j) s += b0 + j < nb ? btot[b0 + j] : 0;
    int total;
    int run = block_exclusive_scan<VSCAN>(s, waves, total);
    for (int j = 0; j < per; ++j)
        if (b0 + j < nb) {
            boff[b0 + j] = run;
            run += btot[b0 + j];
        }
    if (threadIdx.x == 0) hdr[V_TOTAL] = uint32_t(total);
}

// Voxel number of each first point's voxel, stored at its table slot (-1
// when beyond max_voxels).
__global__ __launch_bounds__(VT) void k_vox_number(const uint64_t* __restrict__ table,
                                                   const int32_t* __restrict__ slot, int32_t n,
                                                   const int32_t* __restrict__ boff, int32_t max_voxels,
                                                   int32_t* __restrict__ svid) {
    __shared__ int waves[VT / WAVE];
    const int i = int(blockIdx.x) * VT + int(threadIdx.x);
    const bool f = is_first(table, slot, i, n);
    int total;
    const int vid = boff[blockIdx.x] + block_exclusive_scan<VT>(f ? 1 : 0, waves, total);
    if (f) svid[slot[i]] = vid < max_voxels ? vid : -1;
}

// Sort key of each point: its voxel number, or max_voxels (sorts last) for a
// point outside the box or in a dropped voxel.  Also resets the point ids.
__global__ __launch_bounds__(VT) void k_vox_keys(const int32_t* __restrict__ slot, const int32_t* __restrict__ svid,
                                                 int32_t n, int32_t max_voxels, uint32_t* __restrict__ skey,
                                                 int32_t* __restrict__ pcid) {
    const int i = int(blockIdx.x) * VT + int(threadIdx.x);
    if (i >= n) return;
    const int32_t s = slot[i];
    const int32_t v = s >= 0 ? svid[s] : -1;
    skey[i] = v >= 0 ? uint32_t(v) : uint32_t(max_voxels);
    if (pcid) pcid[i] = -1;
}

// Run [start, end) of every kept voxel in the sorted order.
__global__ __launch_bounds__(VT) void k_vox_segments(const uint32_t* __restrict__ key, int32_t n, int32_t max_voxels,
                                                     int32_t* __restrict__ seg_start, int32_t* __restrict__ seg_end) {
    const int p = int(blockIdx.x) * VT + int(threadIdx.x);
    if (p >= n) return;
    const uint32_t v = key[p];
    if (v >= uint32_t(max_voxels)) return;
    if (p == 0 || key[p - 1] != v) seg_start[v] = p;
    if (p == n - 1 || key[p + 1] != v) seg_end[v] = p + 1;
}

__global__ __launch_bounds__(VT) void k_vox_write(const float* __restrict__ pts, int32_t F,
                                                  const int32_t* __restrict__ order, const uint32_t* __restrict__ keyv,
                                                  const int32_t* __restrict__ seg_start,
                                                  const int32_t* __restrict__ seg_end, const uint32_t* __restrict__ hdr,
                                                  int32_t max_voxels, int32_t max_points, int32_t empty_mean,
                                                  VoxGeom g, float* __restrict__ voxels, int32_t* __restrict__ coords,
                                                  int32_t* __restrict__ num_points, int32_t* __restrict__ pcid) {
    const int64_t t = int64_t(blockIdx.x) * VT + threadIdx.x;
    const int nv = min(int(hdr[V_TOTAL]), max_voxels);
    if (t >= int64_t(nv) * max_points) return;
    const int v = int(t / max_points), s = int(t - int64_t(v) * max_points);
    const int start = seg_start[v];
    const int n = min(seg_end[v] - start, max_points);
    float* dst = voxels + t * F;
    if (s < n) {
        const int pt = order[start + s];
        const float* src = pts + int64_t(pt) * F;
        for (int f = 0; f < F; ++f) dst[f] = src[f];
        if (pcid) pcid[pt] = v;
    } else if (empty_mean) {
        // the mean of the voxel's stored points, summed in slot order
        for (int f = 0; f < F; ++f) {
            float acc = 0.f;
            for (int j = 0; j < n; ++j) acc += pts[int64_t(order[start + j]) * F + f];
            dst[f] = __fdiv_rn(acc, float(n));
        }
    } else {
        for (int f = 0; f < F; ++f) dst[f] = 0.f;
    }
    if (s == 0) {
        num_points[v] = n;
        const uint32_t key = keyv[order[start]];
        const uint32_t x = key % uint32_t(g.ext[0]), yz = key / uint32_t(g.ext[0]);
        coords[3 * v] = int32_t(yz / uint32_t(g.ext[1]));
        coords[3 * v + 1] = int32_t(yz % uint32_t(g.ext[1]));
        coords[3 * v + 2] = int32_t(x);
    }
}

template <typename TT>
__global__ __launch_bounds__(VT) void k_gather_by_id(const void* __restrict__ seg_, int32_t n_vox, int32_t C,
                                                     const int32_t* __restrict__ ids, int32_t n,
                                                     void* __restrict__ out_) {
    using S = typename TT::storage;
    const int cpr = C / TT::E;
    const int64_t g = int64_t(blockIdx.x) * VT + threadIdx.x;
    if (g >= int64_t(n) * cpr) return;
    const int i = int(g / cpr), ch = int(g - int64_t(i) * cpr) * TT::E;
    const int32_t v = ids[i];
    const u32x4 val = (unsigned)v < (unsigned)n_vox ? ld16(static_cast<const S*>(seg_) + int64_t(v) * C + ch) : zero4();
    st16(static_cast<S*>(out_) + int64_t(i) * C + ch, val);
}

// ---------------------------------------------------------------- host side

struct VoxLayout {
    int64_t cap;                       // table slots (power of two >= 2n)
    int passes;                        // radix passes over the voxel numbers
    int64_t nb, nbs, ngs;              // point blocks, radix blocks, radix groups
    int64_t off_table, off_keyv, off_slot, off_btot, off_boff, off_svid, off_keys0, off_sort, off_vals,
        off_hist, off_gsum, off_seg, total;
};

VoxLayout vox_layout(int64_t n, int64_t max_voxels) {
    VoxLayout l{};
    l.cap = 64;
    while (l.cap < 2 * n) l.cap *= 2;
    int bits = 1;
    while ((int64_t(1) << bits) <= max_voxels) ++bits;  // keys run up to max_voxels
    l.passes = (bits + RS_BITS - 1) / RS_BITS;
    l.nb = ceil_div(n, VT);
    l.nbs = ceil_div(n, RS_TILE);
    l.ngs = ceil_div(l.nbs, RS_GROUP);
    int64_t o = 256;  // header
    auto take = [&](int64_t bytes) { const int64_t at = o; o = int64_t(align_up(size_t(o + bytes), 256)); return at; };
    l.off_table = take(l.cap * 8);
    l.off_keyv = take(n * 4);
    l.off_slot = take(n * 4);
    l.off_btot = take(l.nb * 4);
    l.off_boff = take(l.nb * 4);
    l.off_svid = take(l.cap * 4);
    l.off_keys0 = take(n * 4);
    l.off_sort = take(2 * n * 4);      // keys ping-pong
    l.off_vals = take(2 * n * 4);      // values ping-pong
    l.off_hist = take(int64_t(RS_BINS) * l.nbs * 4);
    l.off_gsum = take(int64_t(RS_BINS) * l.ngs * l.passes * 4);
    l.off_seg = take(2 * max_voxels * 4);
    l.total = o;
    return l;
}

spc_status check_geom(const float* vsize, const float* range, VoxGeom* g) {
    if (!vsize || !range) return fail(SPC_ERR_ARG, "vsize_xyz or range_xyz is NULL");
    uint64_t cells = 1;
    for (int a = 0; a < 3; ++a) {
        const double ext = nearbyint((double(range[a + 3]) - double(range[a])) / double(vsize[a]));
        if (!(vsize[a] > 0.f) || !(ext >= 1.0) || ext > 2147483647.0)
            return fail(SPC_ERR_ARG, "axis %d: voxel size %g over [%g, %g) gives no valid grid", a, double(vsize[a]),
                        double(range[a]), double(range[a + 3]));
        g->lo[a] = range[a];
        g->vs[a] = vsize[a];
        g->ext[a] = int32_t(ext);
        cells *= uint64_t(ext);
        if (cells >= 0xFFFFFFFFull) return fail(SPC_ERR_UNSUPPORTED, "the voxel grid exceeds 2^32 - 1 cells");
    }
    return SPC_OK;
}

spc_status check_sizes(int64_t n, int32_t F, int64_t max_voxels, int32_t max_points) {
    if (n < 0 || n >= (int64_t(1) << 31)) return fail(SPC_ERR_ARG, "n_points=%lld out of range", (long long)n);
    if (F < 3 || F > MAX_FEATURES) return fail(SPC_ERR_ARG, "n_features=%d must be in 3..%d", F, MAX_FEATURES);
    if (max_voxels < 1 || max_voxels >= (int64_t(1) << 27))
        return fail(SPC_ERR_ARG, "max_voxels=%lld must be in 1..2^27-1", (long long)max_voxels);
    if (max_points < 1 || max_voxels * max_points >= (int64_t(1) << 31))
        return fail(SPC_ERR_ARG, "max_points=%d: max_voxels * max_points must stay below 2^31", max_points);
    return SPC_OK;
}

}  // namespace
}  // namespace spc

using namespace spc;

extern "C" spc_status spc_point_to_voxel_workspace(int64_t n_points, int32_t n_features, int64_t max_voxels,
                                                   int32_t max_points, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(SPC_ERR_ARG, "bytes is NULL");
    spc_status st = check_sizes(n_points, n_features, max_voxels, max_points);
    if (st != SPC_OK) return st;
    *bytes = size_t(vox_layout(n_points, max_voxels).total);
    return SPC_OK;
}

extern "C" spc_status spc_point_to_voxel(const float* points, int64_t n_points, int32_t n_features,
                                         const float* vsize_xyz, const float* range_xyz, int64_t max_voxels,
                                         int32_t max_points, int32_t empty_mean, float* voxels, int32_t* coords,
                                         int32_t* num_points, int32_t* pc_voxel_id, int64_t* n_voxels, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
    clear_error();
    spc_status st = check_sizes(n_points, n_features, max_voxels, max_points);
    if (st != SPC_OK) return st;
    VoxGeom g;
    st = check_geom(vsize_xyz, range_xyz, &g);
    if (st != SPC_OK) return st;
    if (!n_voxels) return fail(SPC_ERR_ARG, "n_voxels is NULL");
    *n_voxels = 0;
    if (n_points == 0) return SPC_OK;
    if (!points || !voxels || !coords || !num_points) return fail(SPC_ERR_ARG, "an input or output pointer is NULL");
    const VoxLayout l = vox_layout(n_points, max_voxels);
    if (!ws || ws_bytes < size_t(l.total))
        return fail(SPC_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", ws_bytes, (long long)l.total);
    if (!aligned16(ws)) return fail(SPC_ERR_ARG, "the workspace must be 16-byte aligned");

    char* w = static_cast<char*>(ws);
    uint32_t* hdr = reinterpret_cast<uint32_t*>(w);
    uint64_t* table = reinterpret_cast<uint64_t*>(w + l.off_table);
    uint32_t* keyv = reinterpret_cast<uint32_t*>(w + l.off_keyv);
    int32_t* slot = reinterpret_cast<int32_t*>(w + l.off_slot);
    int32_t* btot = reinterpret_cast<int32_t*>(w + l.off_btot);
    int32_t* boff = reinterpret_cast<int32_t*>(w + l.off_boff);
    int32_t* svid = reinterpret_cast<int32_t*>(w + l.off_svid);
    uint32_t* keys0 = reinterpret_cast<uint32_t*>(w + l.off_keys0);
    uint32_t* kbuf[2] = {reinterpret_cast<uint32_t*>(w + l.off_sort),
                         reinterpret_cast<uint32_t*>(w + l.off_sort) + n_points};
    int32_t* vbuf[2] = {reinterpret_cast<int32_t*>(w + l.off_vals), reinterpret_cast<int32_t*>(w + l.off_vals) + n_points};
    int32_t* hist = reinterpret_cast<int32_t*>(w + l.off_hist);
    int32_t* gsum = reinterpret_cast<int32_t*>(w + l.off_gsum);
    int32_t* seg_start = reinterpret_cast<int32_t*>(w + l.off_seg);
    int32_t* seg_end = seg_start + max_voxels;
    const int32_t n = int32_t(n_points), mv = int32_t(max_voxels);

    const int64_t nzero = int64_t(RS_BINS) * l.ngs * l.passes;
    hipLaunchKernelGGL(k_vox_clear, dim3(unsigned(std::min<int64_t>(ceil_div(l.cap / 2, VT), 2048))), dim3(VT), 0,
                       stream, table, l.cap, hdr, gsum, nzero);
    SPC_LAUNCHED("k_vox_clear");
    const dim3 pg(unsigned(l.nb));
    hipLaunchKernelGGL(k_vox_insert, pg, dim3(VT), 0, stream, points, n, n_features, g, table, uint32_t(l.cap - 1),
                       keyv, slot);
    SPC_LAUNCHED("k_vox_insert");
    hipLaunchKernelGGL(k_vox_first, pg, dim3(VT), 0, stream, table, slot, n, btot);
    SPC_LAUNCHED("k_vox_first");
    hipLaunchKernelGGL(k_vox_scan, dim3(1), dim3(VSCAN), 0, stream, btot, int32_t(l.nb), boff, hdr);
    SPC_LAUNCHED("k_vox_scan");
    hipLaunchKernelGGL(k_vox_number, pg, dim3(VT), 0, stream, table, slot, n, boff, mv, svid);
    SPC_LAUNCHED("k_vox_number");
    hipLaunchKernelGGL(k_vox_keys, pg, dim3(VT), 0, stream, slot, svid, n, mv, keys0, pc_voxel_id);
    SPC_LAUNCHED("k_vox_keys");
    const uint32_t* kin = keys0;
    const int32_t* vin = nullptr;  // identity: the point index
    for (int pass = 0; pass < l.passes; ++pass) {
        RsPass P{};
        RsJob& J = P.job[0];
        J.keys_in = kin;
        J.vals_in = vin;
        J.keys_out = kbuf[pass & 1];
        J.vals_out = vbuf[pass & 1];
        J.hist = hist;
        J.gsum = gsum + int64_t(pass) * RS_BINS * l.ngs;
        J.n_dev = nullptr;
        J.cap = n;
        J.rows = n;
        J.nb = int(l.nbs);
        J.ng = int(l.ngs);
        P.shift = RS_BITS * pass;
        hipLaunchKernelGGL(k_rs_hist, dim3(unsigned(l.nbs)), dim3(RS_THREADS), 0, stream, P);
        SPC_LAUNCHED("k_rs_hist");
        hipLaunchKernelGGL(k_rs_scatter, dim3(unsigned(l.nbs)), dim3(RS_THREADS), 0, stream, P);
        SPC_LAUNCHED("k_rs_scatter");
        kin = kbuf[pass & 1];
        vin = vbuf[pass & 1];
    }
    hipLaunchKernelGGL(k_vox_segments, pg, dim3(VT), 0, stream, kin, n, mv, seg_start, seg_end);
    SPC_LAUNCHED("k_vox_segments");
    hipLaunchKernelGGL(k_vox_write, dim3(unsigned(ceil_div(max_voxels * max_points, VT))), dim3(VT), 0, stream, points,
                       n_features, vin, keyv, seg_start, seg_end, hdr, mv, max_points, empty_mean ? 1 : 0, g, voxels,
                       coords, num_points, pc_voxel_id);
    SPC_LAUNCHED("k_vox_write");
    uint32_t total = 0;
    SPC_HIP(hipMemcpyAsync(&total, hdr + V_TOTAL, sizeof(total), hipMemcpyDeviceToHost, stream));
    SPC_HIP(hipStreamSynchronize(stream));
    *n_voxels = std::min<int64_t>(total, max_voxels);
    return SPC_OK;
}

extern "C" spc_status spc_gather_by_voxel_id(spc_dtype dtype, const void* seg_features, int64_t n_voxels,
                                             int32_t C, const int32_t* pc_voxel_id, int64_t n_points, void* out,
                                             hipStream_t stream) {
    clear_error();
    if (dtype != SPC_F32 && dtype != SPC_F16 && dtype != SPC_BF16) return fail(SPC_ERR_ARG, "unknown dtype %d", int(dtype));
    if (C <= 0 || C % 16) return fail(SPC_ERR_UNSUPPORTED, "C=%d: channels must be a positive multiple of 16", C);
    if (n_points < 0 || n_voxels < 0 || n_voxels >= (int64_t(1) << 31) ||
        n_points * (C / (dtype == SPC_F32 ? 4 : 8)) >= (int64_t(1) << 40))
        return fail(SPC_ERR_ARG, "sizes out of range");
    if (n_points == 0) return SPC_OK;
    if (!pc_voxel_id || !out || (n_voxels > 0 && !seg_features))
        return fail(SPC_ERR_ARG, "seg_features, pc_voxel_id or out is NULL");
    for (const void* p : {seg_features, (const void*)pc_voxel_id, (const void*)out})
        if (p && !aligned16(p)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    const int32_t nv = n_voxels > 0 ? int32_t(n_voxels) : 0;
    const int64_t threads = n_points * (C / (dtype == SPC_F32 ? 4 : 8));
    const dim3 grid(unsigned(ceil_div(threads, VT)));
    switch (dtype) {
        case SPC_F32:
            hipLaunchKernelGGL(k_gather_by_id<F32>, grid, dim3(VT), 0, stream, seg_features, nv, C, pc_voxel_id,
                               int32_t(n_points), out);
            break;
        case SPC_F16:
            hipLaunchKernelGGL(k_gather_by_id<F16>, grid, dim3(VT), 0, stream, seg_features, nv, C, pc_voxel_id,
                               int32_t(n_points), out);
            break;
        case SPC_BF16:
            hipLaunchKernelGGL(k_gather_by_id<BF16>, grid, dim3(VT), 0, stream, seg_features, nv, C, pc_voxel_id,
                               int32_t(n_points), out);
            break;
    }
    SPC_LAUNCHED("k_gather_by_id");
    return SPC_OK;
}
