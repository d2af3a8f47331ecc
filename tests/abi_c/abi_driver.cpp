// A caller of libspc that uses nothing but the C ABI of include/spc.h and the
// HIP runtime's C API (no Python, no torch): it reads a submanifold layer from
// a file, builds the kernel map with its processing order, runs the fp32
// forward and writes the map and the outputs back.  The GPU tests run it as a
// child process and compare its results with the oracle.
//
// Input file (little-endian): int32 n, cin, cout, batch, Z, Y, X, ksize; then
// coords int32 [n, 4] (b, z, y, x), feats fp32 [n, cin], weight fp32
// [K, cin, cout], bias fp32 [cout].  Output file: int32 status, then nbr
// int32 [n, K] and out fp32 [n, cout].  Exit status 0 on success.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "spc.h"

namespace {

bool hip_ok(hipError_t e, const char* what) {
    if (e == hipSuccess) return true;
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return false;
}

bool spc_ok(spc_status st, const char* what) {
    if (st == SPC_OK) return true;
    std::fprintf(stderr, "%s: status %d: %s\n", what, int(st), spc_last_error());
    return false;
}

template <typename T>
bool read_n(std::FILE* f, std::vector<T>& v, size_t n) {
    v.resize(n);
    return std::fread(v.data(), sizeof(T), n, f) == n;
}

template <typename T>
T* to_device(const std::vector<T>& v) {
    void* p = nullptr;
    const size_t bytes = v.size() * sizeof(T);
    if (!hip_ok(hipMalloc(&p, bytes > 0 ? bytes : 16), "hipMalloc")) return nullptr;
    if (bytes && !hip_ok(hipMemcpy(p, v.data(), bytes, hipMemcpyHostToDevice), "hipMemcpy")) return nullptr;
    return static_cast<T*>(p);
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s <input file> <output file>\n", argv[0]);
        return 2;
    }
    std::FILE* in = std::fopen(argv[1], "rb");
    if (!in) return 2;
    int32_t hdr[8];
    if (std::fread(hdr, sizeof(int32_t), 8, in) != 8) return 2;
    const int32_t n = hdr[0], cin = hdr[1], cout = hdr[2], k = hdr[7];
    const int32_t K = k * k * k;
    std::vector<int32_t> coords;
    std::vector<float> feats, weight, bias;
    if (!read_n(in, coords, size_t(n) * 4) || !read_n(in, feats, size_t(n) * cin) ||
        !read_n(in, weight, size_t(K) * cin * cout) || !read_n(in, bias, size_t(cout)))
        return 2;
    std::fclose(in);

    spc_geom g{};
    g.batch = hdr[3];
    g.shape[0] = hdr[4];
    g.shape[1] = hdr[5];
    g.shape[2] = hdr[6];
    for (int a = 0; a < 3; ++a) g.ksize[a] = k, g.stride[a] = 1, g.pad[a] = k / 2, g.dil[a] = 1;
    g.subm = 1;
    g.table = SPC_TABLE_HASH;

    size_t ws_bytes = 0;
    if (!spc_ok(spc_kmap_workspace(&g, n, &ws_bytes), "spc_kmap_workspace")) return 1;
    int32_t* d_coords = to_device(coords);
    float* d_feats = to_device(feats);
    float* d_weight = to_device(weight);
    float* d_bias = to_device(bias);
    void *d_nbr = nullptr, *d_order = nullptr, *d_err = nullptr, *d_out = nullptr, *d_ws = nullptr;
    if (!d_coords || !d_feats || !d_weight || !d_bias) return 1;
    if (!hip_ok(hipMalloc(&d_nbr, size_t(n) * K * 4 + 16), "hipMalloc") ||
        !hip_ok(hipMalloc(&d_order, size_t(n) * 4 + 16), "hipMalloc") ||
        !hip_ok(hipMalloc(&d_err, 16), "hipMalloc") ||
        !hip_ok(hipMalloc(&d_out, size_t(n) * cout * 4 + 16), "hipMalloc") ||
        !hip_ok(hipMalloc(&d_ws, ws_bytes > 0 ? ws_bytes : 16), "hipMalloc"))
        return 1;
    hipStream_t stream = nullptr;
    if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;

    int64_t n_out = 0;
    if (!spc_ok(spc_build_kmap(&g, d_coords, n, nullptr, 0, &n_out, static_cast<int32_t*>(d_nbr), nullptr, nullptr,
                               nullptr, nullptr, 0, static_cast<int32_t*>(d_order), nullptr,
                               static_cast<int32_t*>(d_err), d_ws, ws_bytes, stream),
                "spc_build_kmap"))
        return 1;
    if (!spc_ok(spc_subm_conv_fwd(SPC_F32, d_feats, n, cin, d_weight, K, cout, d_bias, static_cast<int32_t*>(d_nbr),
                                  static_cast<int32_t*>(d_order), d_out, stream),
                "spc_subm_conv_fwd"))
        return 1;
    if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;

    int32_t err = 0;
    std::vector<int32_t> nbr(size_t(n) * K);
    std::vector<float> out(size_t(n) * cout);
    if (!hip_ok(hipMemcpy(&err, d_err, 4, hipMemcpyDeviceToHost), "hipMemcpy") ||
        !hip_ok(hipMemcpy(nbr.data(), d_nbr, nbr.size() * 4, hipMemcpyDeviceToHost), "hipMemcpy") ||
        !hip_ok(hipMemcpy(out.data(), d_out, out.size() * 4, hipMemcpyDeviceToHost), "hipMemcpy"))
        return 1;
    std::FILE* o = std::fopen(argv[2], "wb");
    if (!o) return 2;
    std::fwrite(&err, sizeof(int32_t), 1, o);
    std::fwrite(nbr.data(), sizeof(int32_t), nbr.size(), o);
    std::fwrite(out.data(), sizeof(float), out.size(), o);
    std::fclose(o);
    bool freed = true;
    for (void* p : {static_cast<void*>(d_coords), static_cast<void*>(d_feats), static_cast<void*>(d_weight),
                    static_cast<void*>(d_bias), d_nbr, d_order, d_err, d_out, d_ws})
        freed = hip_ok(hipFree(p), "hipFree") && freed;
    freed = hip_ok(hipStreamDestroy(stream), "hipStreamDestroy") && freed;
    return freed ? 0 : 1;
}
