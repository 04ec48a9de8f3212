// Calls the C-ABI library from a plain host program: no Python, no torch.
//
//   c_abi_driver <dir> <B> <H> <N> <D> <causal> <softmax_scale>
//
// Reads <dir>/{q,k,v,do}.bin (raw 16-bit bf16, [B, H, N, D] each), puts them
// in device memory from hipMalloc, runs fa_fwd and then fa_bwd (with a
// workspace of fa_bwd_workspace_size bytes) on a stream of its own, and writes
// <dir>/{o,dq,dk,dv}.bin (bf16) and <dir>/lse.bin (fp32).  Every status is
// checked and printed through fa_status_string; the exit code is 0 only when
// all calls succeed.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "fa.h"

namespace {

bool read_file(const std::string& path, std::vector<uint16_t>& out, size_t n) {
    FILE* f = std::fopen(path.c_str(), "rb");
    if (!f) return false;
    out.resize(n);
    const size_t got = std::fread(out.data(), sizeof(uint16_t), n, f);
    std::fclose(f);
    return got == n;
}

template <typename T>
bool write_file(const std::string& path, const std::vector<T>& v) {
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f) return false;
    const size_t put = std::fwrite(v.data(), sizeof(T), v.size(), f);
    std::fclose(f);
    return put == v.size();
}

#define HIP_OK(call)                                                             \
    do {                                                                         \
        hipError_t e_ = (call);                                                  \
        if (e_ != hipSuccess) {                                                  \
            std::fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));      \
            return 2;                                                            \
        }                                                                        \
    } while (0)

#define FA_OK_OR_FAIL(call)                                                      \
    do {                                                                         \
        int s_ = (call);                                                         \
        std::printf("%s -> %s\n", #call, fa_status_string(s_));                  \
        if (s_ != FA_OK) return 3;                                               \
    } while (0)

}  // namespace

int main(int argc, char** argv) {
    if (argc != 8) {
        std::fprintf(stderr, "usage: %s dir B H N D causal softmax_scale\n", argv[0]);
        return 1;
    }
    const std::string dir = argv[1];
    const int B = std::atoi(argv[2]), H = std::atoi(argv[3]), N = std::atoi(argv[4]);
    const int D = std::atoi(argv[5]), causal = std::atoi(argv[6]);
    const size_t n = (size_t)B * H * N * D, rows = (size_t)B * H * N;
    const float scale = std::strtof(argv[7], nullptr);

    std::vector<uint16_t> h_q, h_k, h_v, h_do;
    if (!read_file(dir + "/q.bin", h_q, n) || !read_file(dir + "/k.bin", h_k, n) ||
        !read_file(dir + "/v.bin", h_v, n) || !read_file(dir + "/do.bin", h_do, n)) {
        std::fprintf(stderr, "cannot read the inputs in %s\n", dir.c_str());
        return 1;
    }

    void *q, *k, *v, *o, *dout, *dq, *dk, *dv, *ws;
    float* lse;
    const size_t bytes = n * sizeof(uint16_t);
    HIP_OK(hipMalloc(&q, bytes));
    HIP_OK(hipMalloc(&k, bytes));
    HIP_OK(hipMalloc(&v, bytes));
    HIP_OK(hipMalloc(&o, bytes));
    HIP_OK(hipMalloc(&dout, bytes));
    HIP_OK(hipMalloc(&dq, bytes));
    HIP_OK(hipMalloc(&dk, bytes));
    HIP_OK(hipMalloc(&dv, bytes));
    HIP_OK(hipMalloc(&lse, rows * sizeof(float)));
    const size_t ws_bytes = fa_bwd_workspace_size(B, H, N, D);
    std::printf("fa_bwd_workspace_size(%d, %d, %d, %d) = %zu\n", B, H, N, D, ws_bytes);
    if (ws_bytes == 0) return 3;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    HIP_OK(hipMemcpy(q, h_q.data(), bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, h_k.data(), bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, h_v.data(), bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dout, h_do.data(), bytes, hipMemcpyHostToDevice));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    FA_OK_OR_FAIL(fa_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, stream));
    FA_OK_OR_FAIL(fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, B, H, N, D, scale,
                         causal, stream));
    HIP_OK(hipStreamSynchronize(stream));

    std::vector<uint16_t> h_o(n), h_dq(n), h_dk(n), h_dv(n);
    std::vector<float> h_lse(rows);
    HIP_OK(hipMemcpy(h_o.data(), o, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_dq.data(), dq, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_dk.data(), dk, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_dv.data(), dv, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_lse.data(), lse, rows * sizeof(float), hipMemcpyDeviceToHost));
    const bool ok = write_file(dir + "/o.bin", h_o) && write_file(dir + "/lse.bin", h_lse) &&
                    write_file(dir + "/dq.bin", h_dq) && write_file(dir + "/dk.bin", h_dk) &&
                    write_file(dir + "/dv.bin", h_dv);
    HIP_OK(hipStreamDestroy(stream));
    for (void* p : {q, k, v, o, dout, dq, dk, dv, ws}) HIP_OK(hipFree(p));
    HIP_OK(hipFree(lse));
    std::printf(ok ? "c_abi_driver ok\n" : "c_abi_driver: cannot write the outputs\n");
    return ok ? 0 : 1;
}
