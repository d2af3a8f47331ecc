// Fused implicit-GEMM sparse convolution: gather -> MFMA -> output-stationary
// accumulate, one kernel per call.
//
//   y[r, :] = bias + sum_k  x[map[k][r], :] @ B_k          (map[k][r] >= 0)
//
// covers the submanifold and strided forward (B_k = W[k], the MLX
// sparse/conv.py page's formula), the per-voxel k=1 layer (identity map) and
// dinput (B_k = W[k]^T or W[K-1-k]^T, gathered from dout through the
// input-stationary map).  Absent neighbours contribute nothing, like the MLX
// page's appended zero row, but here a missing row is a predicated-off load
// that leaves a zero fragment.
//
// Work split (CDNA4, 64-lane waves): a workgroup of 4 waves owns BM = 4*RB*16
// output rows and BN = NB*16 output channels.  For each offset that has at
// least one hit among its rows it stages B_k's [CK x BN] slab in LDS (in the
// 16-byte MFMA fragment layout, transposing W on the fly when needed), and
// every wave multiplies its gathered rows, loaded straight from global memory
// into registers as 16-byte fragments, with v_mfma_f32_16x16x32_{bf16,f16}
// (or v_mfma_f32_16x16x4_f32).  The fp32 accumulators stay in registers for
// the whole offset loop; each output row is written once, with the bias added
// and one rounding, so there are no atomics and the result is deterministic.
#include <algorithm>

#include "common.h"

namespace spc {
namespace {

constexpr int CT = 256;          // threads per workgroup
constexpr int NW = CT / WAVE;    // waves per workgroup
constexpr int KTILE = 32;        // offsets whose map rows are staged at once

struct ConvArgs {
    const void* x;       // gathered operand [n_src, CK]
    const void* w;       // weights [K, cin, cout]
    const float* bias;   // [CN] or NULL
    const int32_t* map;  // [K, n_rows] or NULL (identity, K == 1)
    void* y;             // [n_rows, CN]
    int32_t n_rows, n_src, K;
    int32_t CK, CN;      // contraction / output channels
    int32_t cin, cout;   // weight dims
    int32_t w_rev;       // slab of offset k is W[K-1-k]
    int32_t kch;         // 16-byte chunks along CK, padded to a multiple of 4
};

// LDS slab layout: chunk row kb (16 bytes of CK per output channel) has BN
// entries of 16 bytes plus 16 bytes of padding, which keeps both the staging
// writes and the fragment reads free of bank conflicts.
template <int BN>
__device__ __forceinline__ int slab_off(int kb, int n) {
    return kb * (BN * 16 + 16) + n * 16;
}

// Stages B_k (slab ws of W) into LDS.  TRANS: B[kk][n] = W[ws][kk][n] (the
// forward; W rows are output channels apart, so E x E blocks are transposed
// in registers).  !TRANS: B[kk][n] = W[ws][n][kk] (dinput; already
// contraction-contiguous).  Chunks beyond CK are zero.
template <typename TT, int BN, bool TRANS>
__device__ __forceinline__ void stage_slab(char* lds, const ConvArgs& a, int ws, int col0) {
    using S = typename TT::storage;
    constexpr int E = TT::E;
    const S* w = static_cast<const S*>(a.w);
    const int ckc = a.CK / E;  // real chunks
    if (TRANS) {
        constexpr int NBK = BN / E;
        for (int idx = threadIdx.x; idx < a.kch * NBK; idx += CT) {
            const int kb = idx % a.kch, nbk = idx / a.kch;
            u32x4 in[E];
            if (kb < ckc) {
                const S* src = w + (int64_t(ws) * a.cin + kb * E) * a.cout + col0 + nbk * E;
#pragma unroll
                for (int e = 0; e < E; ++e) in[e] = ld16(src + int64_t(e) * a.cout);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) in[e] = zero4();
            }
            if constexpr (E == 8) {
                typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
                u16x8 v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(u16x8, in[e]);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    u16x8 o = {v[0][j], v[1][j], v[2][j], v[3][j], v[4][j], v[5][j], v[6][j], v[7][j]};
                    st16(lds + slab_off<BN>(kb, nbk * 8 + j), __builtin_bit_cast(u32x4, o));
                }
            } else {
                const uint32_t m[4][4] = {{in[0].x, in[0].y, in[0].z, in[0].w},
                                          {in[1].x, in[1].y, in[1].z, in[1].w},
                                          {in[2].x, in[2].y, in[2].z, in[2].w},
                                          {in[3].x, in[3].y, in[3].z, in[3].w}};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    st16(lds + slab_off<BN>(kb, nbk * 4 + j), u32x4{m[0][j], m[1][j], m[2][j], m[3][j]});
            }
        }
    } else {
        for (int idx = threadIdx.x; idx < a.kch * BN; idx += CT) {
            const int kb = idx % a.kch, n = idx / a.kch;
            u32x4 v = zero4();
            if (kb < ckc) v = ld16(w + (int64_t(ws) * a.cin + col0 + n) * a.cout + kb * E);
            st16(lds + slab_off<BN>(kb, n), v);
        }
    }
}

template <typename TT, int RB, int NB, bool TRANS, int KCMAX>
__global__ __launch_bounds__(CT) void k_conv(ConvArgs a) {
    using S = typename TT::storage;
    constexpr int E = TT::E;
    constexpr int BN = NB * 16;
    constexpr int BM = NW * RB * 16;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char* slab = lds;
    int32_t* tile = reinterpret_cast<int32_t*>(lds + a.kch * (BN * 16 + 16));   // [KTILE][BM]
    int32_t* flags = tile + KTILE * BM;                                            // [KTILE]

    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = blockIdx.x * BM, col0 = blockIdx.y * BN;
    const int KC = a.kch / 4;  // MFMA steps along CK
    const S* x = static_cast<const S*>(a.x);

    f32x4_t acc[RB][NB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int kt0 = 0; kt0 < a.K; kt0 += KTILE) {
        const int kt = min(KTILE, a.K - kt0);
        __syncthreads();  // earlier readers of tile / flags / slab are done
        if (threadIdx.x < KTILE) flags[threadIdx.x] = 0;
        __syncthreads();
        for (int idx = threadIdx.x; idx < kt * BM; idx += CT) {
            const int k = idx / BM, r = idx - k * BM, row = row0 + r;
            int32_t v = -1;
            if (row < a.n_rows) v = a.map ? a.map[int64_t(kt0 + k) * a.n_rows + row] : row;
            if ((unsigned)v >= (unsigned)a.n_src) v = -1;
            tile[idx] = v;
            if (v >= 0) flags[k] = 1;
        }
        __syncthreads();
        for (int k = 0; k < kt; ++k) {
            if (!flags[k]) continue;  // no row of this workgroup reads offset k
            const int kg = kt0 + k;
            // gather this wave's rows (in flight while the slab is staged)
            u32x4 af[RB][KCMAX];
            bool any = false;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int32_t src = tile[k * BM + (wave * RB + rb) * 16 + lr];
                any |= src >= 0;
                const S* p = x + int64_t(src) * a.CK + lg * E;
#pragma unroll
                for (int kc = 0; kc < KCMAX; ++kc) {
                    af[rb][kc] = zero4();
                    if (kc < KC && src >= 0 && (kc * 4 + lg) * E < a.CK) af[rb][kc] = ld16(p + kc * 4 * E);
                }
            }
            __syncthreads();  // the previous slab is no longer read
            stage_slab<TT, BN, TRANS>(slab, a, a.w_rev ? a.K - 1 - kg : kg, col0);
            __syncthreads();
            if (!__any(any)) continue;  // wave-uniform: none of this wave's rows hit
#pragma unroll
            for (int kc = 0; kc < KCMAX; ++kc) {
                if (kc >= KC) break;
                u32x4 bf[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) bf[nb] = ld16(slab + slab_off<BN>(kc * 4 + lg, nb * 16 + lr));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) acc[rb][nb] = mfma16<TT>(bf[nb], af[rb][kc], acc[rb][nb]);
            }
        }
    }

    // epilogue: D[channel][row] per 16x16 tile; this lane holds channels
    // lg*4 .. lg*4+3 of row lr, so each store is 4 consecutive channels
    S* y = static_cast<S*>(a.y);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = row0 + (wave * RB + rb) * 16 + lr;
        if (row >= a.n_rows) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int ch = col0 + nb * 16 + lg * 4;
            f32x4_t v = acc[rb][nb];
            if (a.bias) {
                const f32x4_t b = *reinterpret_cast<const f32x4_t*>(a.bias + ch);
                v += b;
            }
            store4<TT>(y + int64_t(row) * a.CN + ch, v);
        }
    }
}

constexpr int RB_DEFAULT = 2;

template <typename TT, int NB, bool TRANS, int KCMAX>
spc_status launch_conv_nb(const ConvArgs& a, hipStream_t stream) {
    constexpr int BN = NB * 16;
    constexpr int BM = NW * RB_DEFAULT * 16;
    auto kern = k_conv<TT, RB_DEFAULT, NB, TRANS, KCMAX>;
    const size_t lds = size_t(a.kch) * (BN * 16 + 16) + size_t(KTILE) * BM * 4 + KTILE * 4;
    if (lds > 160 * 1024) return fail(SPC_ERR_UNSUPPORTED, "LDS tile of %zu bytes exceeds 160 KiB", lds);
    if (lds > 64 * 1024) SPC_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)));
    dim3 grid(unsigned(ceil_div(a.n_rows, BM)), unsigned(a.CN / BN));
    hipLaunchKernelGGL(kern, grid, dim3(CT), lds, stream, a);
    SPC_LAUNCHED("k_conv");
    return SPC_OK;
}

template <typename TT, bool TRANS, int KCMAX>
spc_status launch_conv_k(const ConvArgs& a, hipStream_t stream) {
    const int blocks = a.CN / 16;
    if (blocks % 8 == 0) return launch_conv_nb<TT, 8, TRANS, KCMAX>(a, stream);
    if (blocks % 6 == 0) return launch_conv_nb<TT, 6, TRANS, KCMAX>(a, stream);
    if (blocks % 4 == 0) return launch_conv_nb<TT, 4, TRANS, KCMAX>(a, stream);
    if (blocks % 3 == 0) return launch_conv_nb<TT, 3, TRANS, KCMAX>(a, stream);
    if (blocks % 2 == 0) return launch_conv_nb<TT, 2, TRANS, KCMAX>(a, stream);
    return launch_conv_nb<TT, 1, TRANS, KCMAX>(a, stream);
}

template <typename TT, bool TRANS>
spc_status launch_conv_t(ConvArgs& a, hipStream_t stream) {
    constexpr int E = TT::E;
    a.kch = int(ceil_div(a.CK / E, 4) * 4);
    const int KC = a.kch / 4;
    if (KC <= 4) return launch_conv_k<TT, TRANS, 4>(a, stream);
    if (KC <= 8) return launch_conv_k<TT, TRANS, 8>(a, stream);
    return fail(SPC_ERR_UNSUPPORTED, "contraction of %d channels exceeds %d for this dtype", a.CK, 8 * 4 * E);
}

spc_status run_conv(spc_dtype dt, ConvArgs& a, bool trans, hipStream_t stream) {
    if (a.n_rows == 0) return SPC_OK;
    switch (dt) {
        case SPC_F32: return trans ? launch_conv_t<F32, true>(a, stream) : launch_conv_t<F32, false>(a, stream);
        case SPC_F16: return trans ? launch_conv_t<F16, true>(a, stream) : launch_conv_t<F16, false>(a, stream);
        case SPC_BF16: return trans ? launch_conv_t<BF16, true>(a, stream) : launch_conv_t<BF16, false>(a, stream);
    }
    return fail(SPC_ERR_ARG, "unknown dtype %d", int(dt));
}

spc_status check_common(spc_dtype dt, int64_t n_rows, int64_t n_src, int32_t cin, int32_t cout, int32_t K,
                        const void* x, const void* w, const float* bias, const void* y, const int32_t* map,
                        bool map_required) {
    if (dt != SPC_F32 && dt != SPC_F16 && dt != SPC_BF16) return fail(SPC_ERR_ARG, "unknown dtype %d", int(dt));
    if (n_rows < 0 || n_rows >= (int64_t(1) << 31) || n_src < 0 || n_src >= (int64_t(1) << 31))
        return fail(SPC_ERR_ARG, "row counts out of range");
    if (cin <= 0 || cout <= 0 || cin % 16 || cout % 16)
        return fail(SPC_ERR_UNSUPPORTED, "cin=%d cout=%d: channel counts must be positive multiples of 16", cin, cout);
    if (K <= 0 || K > 343) return fail(SPC_ERR_ARG, "K=%d must be in 1..343", K);
    if (n_rows > 0) {
        if (!w || !y) return fail(SPC_ERR_ARG, "weight or output pointer is NULL");
        if (n_src > 0 && !x) return fail(SPC_ERR_ARG, "input pointer is NULL");
        if (map_required && !map) return fail(SPC_ERR_ARG, "map is NULL");
    }
    const void* ptrs[] = {x, w, bias, y, map};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    return SPC_OK;
}

}  // namespace
}  // namespace spc

using namespace spc;

extern "C" spc_status spc_subm_conv_fwd(spc_dtype dtype, const void* feats, int64_t n, int32_t cin,
                                        const void* weight, int32_t K, int32_t cout, const float* bias,
                                        const int32_t* nbr, void* out, hipStream_t stream) {
    clear_error();
    spc_status st = check_common(dtype, n, n, cin, cout, K, feats, weight, bias, out, nbr, K != 1);
    if (st != SPC_OK) return st;
    ConvArgs a{feats, weight, bias, K == 1 ? nbr : nbr, out, int32_t(n), int32_t(n), K, cin, cout, cin, cout, 0, 0};
    return run_conv(dtype, a, true, stream);
}

extern "C" spc_status spc_sparse_conv_fwd(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin,
                                          const void* weight, int32_t K, int32_t cout, const float* bias,
                                          const int32_t* nbr_out, int64_t n_out, void* out, hipStream_t stream) {
    clear_error();
    spc_status st = check_common(dtype, n_out, n_in, cin, cout, K, feats, weight, bias, out, nbr_out, true);
    if (st != SPC_OK) return st;
    ConvArgs a{feats, weight, bias, nbr_out, out, int32_t(n_out), int32_t(n_in), K, cin, cout, cin, cout, 0, 0};
    return run_conv(dtype, a, true, stream);
}

extern "C" spc_status spc_conv_bwd_input(spc_dtype dtype, const void* dout, int64_t n_out, int32_t cout,
                                         const void* weight, int32_t K, int32_t cin, const int32_t* map,
                                         int32_t map_is_subm, int64_t n_in, void* din, hipStream_t stream) {
    clear_error();
    const bool identity = (K == 1 && map == nullptr);
    spc_status st = check_common(dtype, n_in, n_out, cin, cout, K, dout, weight, nullptr, din, map, !identity);
    if (st != SPC_OK) return st;
    if ((map_is_subm || identity) && n_out != n_in)
        return fail(SPC_ERR_ARG, "submanifold dinput needs n_out == n_in (%lld vs %lld)", (long long)n_out, (long long)n_in);
    // din rows gather dout rows: contraction over cout, output channels cin
    ConvArgs a{dout, weight, nullptr, map, din, int32_t(n_in), int32_t(n_out), K, cout, cin, cin, cout,
               map_is_subm ? 1 : 0, 0};
    return run_conv(dtype, a, false, stream);
}
