// abi_check -- drives libgqa through its C ABI (include/gqa.h) from native
// code, with the HIP runtime only: no Python, no torch.  Test helper.
//
//   abi_check refusals
//       Host-side behaviour with no GPU work: refused arguments return their
//       codes before any launch, and the host helpers reproduce the pages'
//       tables (head map and window start of "Extend the existing full and
//       cached attention paths", the cache size of the worked example in
//       "How do you implement grouped query attention (GQA)?").
//
//   abi_check gpu DIR B C Hq Hkv d window
//       Reads bf16 inputs written by the caller from DIR (q.bin [B,Hq,d],
//       qp.bin [B,Hq,C,d], k.bin and v.bin [B,Hkv,C,d], seqlens.bin [B]
//       int32), runs gqa_decode (q against the cache) and gqa_prefill (qp,
//       T = C) on a stream of its own with a workspace sized by
//       gqa_decode_workspace_bytes, and writes out_decode.bin [B,Hq,d] and
//       out_prefill.bin [B,C,Hq,d] (bf16 bits) back to DIR.
//
// Exit status 0 on success; 1 with a message on stderr otherwise.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "gqa.h"

namespace {

int fail(const char *what) {
    std::fprintf(stderr, "abi_check: %s\n", what);
    return 1;
}

#define EXPECT(cond, what)                                                                   \
    do {                                                                                     \
        if (!(cond))                                                                         \
            return fail(what);                                                               \
    } while (0)

#define HIP_OK(call)                                                                         \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess) {                                                              \
            std::fprintf(stderr, "abi_check: %s: %s\n", #call, hipGetErrorString(e_));      \
            return 1;                                                                        \
        }                                                                                    \
    } while (0)

bool read_file(const std::string &path, void *dst, size_t bytes) {
    FILE *f = std::fopen(path.c_str(), "rb");
    if (!f)
        return false;
    const size_t got = std::fread(dst, 1, bytes, f);
    std::fclose(f);
    return got == bytes;
}

bool write_file(const std::string &path, const void *src, size_t bytes) {
    FILE *f = std::fopen(path.c_str(), "wb");
    if (!f)
        return false;
    const size_t put = std::fwrite(src, 1, bytes, f);
    return std::fclose(f) == 0 && put == bytes;
}

int refusals() {
    // Stand-in device pointers: every call below is refused by a host-side
    // check before anything could dereference them.
    void *P = reinterpret_cast<void *>(uintptr_t{4096});
    const int32_t B = 2, C = 8000, Hq = 8, Hkv = 2, d = 128; // long enough to be split
    EXPECT(gqa_decode(P, P, P, P, nullptr, B, C, Hq, Hkv, d, 0, 0.5f, GQA_BF16, P, 1 << 20,
                      nullptr) == GQA_ERR_ZERO_WINDOW,
           "window 0 is not refused");
    EXPECT(gqa_decode(P, P, P, P, nullptr, B, C, 6, 4, d, -1, 0.5f, GQA_BF16, P, 1 << 20,
                      nullptr) == GQA_ERR_HEADS,
           "Hq % Hkv != 0 is not refused");
    EXPECT(gqa_prefill(P, P, P, P, nullptr, B, C + 1, C, Hq, Hkv, d, -1, 0.5f, GQA_BF16,
                       nullptr) == GQA_ERR_SHAPE,
           "T > C is not refused");
    EXPECT(gqa_decode(P, P, P, P, nullptr, B, GQA_MAX_CELLS + 1, Hq, Hkv, d, -1, 0.5f,
                      GQA_BF16, P, 1 << 20, nullptr) == GQA_ERR_SHAPE,
           "a cache longer than GQA_MAX_CELLS is not refused");
    const size_t need = gqa_decode_workspace_bytes(B, C, Hq, Hkv, d, -1, GQA_BF16);
    EXPECT(need > 0, "no workspace for the split decode");
    EXPECT(gqa_decode(P, P, P, P, nullptr, B, C, Hq, Hkv, d, -1, 0.5f, GQA_BF16, P, need - 1,
                      nullptr) == GQA_ERR_WORKSPACE,
           "a short workspace is not refused");
    EXPECT(gqa_decode(P, P, P, P, nullptr, B, C, Hq, Hkv, d, -1, 0.5f, 7, P, need, nullptr) ==
               GQA_ERR_DTYPE,
           "an unknown dtype is not refused");
    // a matrix-core shape with a pointer aligned to 2 bytes but not to 16
    void *P2 = reinterpret_cast<void *>(uintptr_t{4096 + 2});
    EXPECT(gqa_decode(P2, P, P, P, nullptr, B, C, Hq, Hkv, d, -1, 0.5f, GQA_BF16, P, need,
                      nullptr) == GQA_ERR_ALIGN,
           "a misaligned matrix-core decode is not refused");
    EXPECT(gqa_prefill(P, P, P2, P, nullptr, 1, 64, 64, Hq, Hkv, d, -1, 0.5f, GQA_BF16,
                       nullptr) == GQA_ERR_ALIGN,
           "a misaligned matrix-core prefill is not refused");
    EXPECT(gqa_decode_workspace_bytes(B, 64, Hq, Hkv, d, -1, GQA_BF16) == 0,
           "a short cache (no split) asks for a workspace");
    // head map 8/2 -> 0,0,0,0,1,1,1,1; invalid inputs give -1
    for (int h = 0; h < 8; ++h)
        EXPECT(gqa_kv_head_for_query(h, 8, 2) == h / 4, "head map 8/2");
    EXPECT(gqa_kv_head_for_query(0, 6, 4) == -1, "head map 6/4 is not refused");
    // window start: cell 4 with segment start 2 and window 2 -> 3; w = 0 -> -1
    EXPECT(gqa_window_start(4, 2, 2) == 3 && gqa_window_start(5, 5, 2) == 5, "window start");
    EXPECT(gqa_window_start(3, 0, 0) == -1, "zero window start is not refused");
    // 32 layers x 8 KV heads x d = 128 in fp16 at 8000 tokens: 1,000 MiB
    uint64_t bytes = 0;
    EXPECT(gqa_kv_cache_bytes(32, 1, 8000, 8, 128, 2, &bytes) == GQA_OK &&
               bytes == 1048576000ull,
           "cache bytes of the worked example");
    EXPECT(gqa_status_string(GQA_ERR_ZERO_WINDOW) != nullptr, "status string");
    std::printf("refusals ok\n");
    return 0;
}

int gpu(const std::string &dir, int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t d,
        int32_t window) {
    const size_t nq = (size_t)B * Hq * d, nqp = (size_t)B * Hq * C * d;
    const size_t nkv = (size_t)B * Hkv * C * d;
    std::vector<uint16_t> q(nq), qp(nqp), k(nkv), v(nkv), od(nq), op(nqp);
    std::vector<int32_t> sl(B);
    EXPECT(read_file(dir + "/q.bin", q.data(), nq * 2) &&
               read_file(dir + "/qp.bin", qp.data(), nqp * 2) &&
               read_file(dir + "/k.bin", k.data(), nkv * 2) &&
               read_file(dir + "/v.bin", v.data(), nkv * 2) &&
               read_file(dir + "/seqlens.bin", sl.data(), (size_t)B * 4),
           "cannot read the inputs");
    for (int32_t b = 0; b < B; ++b)
        EXPECT(sl[b] >= 0 && sl[b] <= C, "a length outside 0..C");

    void *dq, *dqp, *dk, *dv, *dod, *dop, *dws;
    int32_t *dsl;
    const size_t ws = gqa_decode_workspace_bytes(B, C, Hq, Hkv, d, window, GQA_BF16);
    HIP_OK(hipMalloc(&dq, nq * 2));
    HIP_OK(hipMalloc(&dqp, nqp * 2));
    HIP_OK(hipMalloc(&dk, nkv * 2));
    HIP_OK(hipMalloc(&dv, nkv * 2));
    HIP_OK(hipMalloc(&dod, nq * 2));
    HIP_OK(hipMalloc(&dop, nqp * 2));
    HIP_OK(hipMalloc(&dws, ws > 0 ? ws : 256));
    HIP_OK(hipMalloc(&dsl, (size_t)B * 4));
    HIP_OK(hipMemcpy(dq, q.data(), nq * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dqp, qp.data(), nqp * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk, k.data(), nkv * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, v.data(), nkv * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dsl, sl.data(), (size_t)B * 4, hipMemcpyHostToDevice));

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    const float scale = 1.0f / std::sqrt((float)d);
    int rc = gqa_decode(dq, dk, dv, dod, dsl, B, C, Hq, Hkv, d, window, scale, GQA_BF16, dws,
                        ws, s);
    if (rc != GQA_OK) {
        std::fprintf(stderr, "abi_check: gqa_decode: %s\n", gqa_status_string(rc));
        return 1;
    }
    rc = gqa_prefill(dqp, dk, dv, dop, dsl, B, C, C, Hq, Hkv, d, window, scale, GQA_BF16, s);
    if (rc != GQA_OK) {
        std::fprintf(stderr, "abi_check: gqa_prefill: %s\n", gqa_status_string(rc));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(od.data(), dod, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(op.data(), dop, nqp * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipStreamDestroy(s));
    for (void *p : {dq, dqp, dk, dv, dod, dop, dws})
        HIP_OK(hipFree(p));
    HIP_OK(hipFree(dsl));
    EXPECT(write_file(dir + "/out_decode.bin", od.data(), nq * 2) &&
               write_file(dir + "/out_prefill.bin", op.data(), nqp * 2),
           "cannot write the outputs");
    std::printf("gpu ok: workspace %zu bytes\n", ws);
    return 0;
}

} // namespace

int main(int argc, char **argv) {
    if (argc >= 2 && std::string(argv[1]) == "refusals")
        return refusals();
    if (argc == 9 && std::string(argv[1]) == "gpu")
        return gpu(argv[2], std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                   std::atoi(argv[6]), std::atoi(argv[7]), std::atoi(argv[8]));
    std::fprintf(stderr, "usage: abi_check refusals | abi_check gpu DIR B C Hq Hkv d window\n");
    return 2;
}
